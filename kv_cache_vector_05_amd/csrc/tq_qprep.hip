// Query preparation for the integer-MFMA logit scan (tq_scan.hip) and the
// fused decode (tq_decode.hip) (tambur post: logits straight from quantised
// keys; iaemfoco post, "TurboQuant: Uma Nova Abordagem" and itstec post, "Por
// dentro do processo de compressao KV": the one-bit QJL correction):
//     q' = Pi RoPE(q),  s = S q'  (s = q' with the sign correction of the
//     TurboESM summary, technical section 2).
// Both are turned into fixed-point integers with one power-of-two scale per
// query (28 bits, |X| <= 2^26) and split into four balanced base-128 int8
// digits, the rows of the scan's and the decode's MFMA A operands; the scale
// and the exact sum of the fixed-point s values go beside them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

// Fixed point with four balanced base-128 digits: returns the shift sh with
// x ~= X * 2^-sh, |X| <= 2^26, and writes the digits (most significant first).
__device__ __forceinline__ int fixed_shift(float amax) {
    if (!(amax > 0.0f)) return 0;
    int e;
    frexpf(amax, &e);
    return 26 - e;
}
__device__ __forceinline__ long long to_fixed(float x, int sh) { return llrint(ldexp((double)x, sh)); }
__device__ __forceinline__ void digits4(long long X, int8_t d[4]) {
#pragma unroll
    for (int k = 3; k >= 1; --k) {
        long long r = ((X + 64) & 127) - 64;
        d[k] = (int8_t)r;
        X = (X - r) >> 7;
    }
    d[0] = (int8_t)X;
}

struct QDig {
    const void* q;
    int32_t bf16, Hq, L_cap, m, sdw, ncs;
    int64_t rows;     // B * Hq
    int32_t norot;    // Pi = I: q' = RoPE(q)
    int32_t s_ident;  // S = I (sign correction): s = q'
    const int32_t* seq_len;
    const int32_t* q_pos;
    const float* rope_cos;
    const float* rope_sin;
    const float* sigma;
    const float* sketch_t;  // S^T [D][m]
    int8_t* qd;      // [rows*4][D]  digits of q' (digit rows 4*row + a)
    int8_t* sd;      // [rows*4][sdw] digits of s in MFMA slot order
    float* scale;    // [rows][3]    shift(q'), shift(s), sum of the fixed-point s values
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// One workgroup per query row.  Every thread first issues its loads: its
// share of S^T (thread (part, l) sums sketch row l over one of 256/m
// coordinate ranges, so each S entry is read once and a wave's loads are
// contiguous), and wave 0 the query, its RoPE row and the signs.  Wave 0 then
// applies RoPE, the sign flips, the Walsh-Hadamard transform (lane l holds
// coordinates l + 64 v: RoPE's pairs and the butterflies are in-lane or one
// cross-lane exchange) and 1/sqrt(d), and writes q' and its digits; after a
// barrier every thread forms its partial sum of s = S q', and after another
// the threads of the first m sum the parts, and wave 0 takes s's scale, the
// exact sum of its fixed-point values and its digits in MFMA slot order.
template <int D, int M>
__global__ __launch_bounds__(256) void qprep_digits_kernel(QDig p) {
    constexpr int VPL = D / 64;
    constexpr int NT = M > 0 ? 256 / M : 1;  // parts per sketch row (M divides 256)
    constexpr int NI = D / NT;               // S^T entries per thread
    __shared__ float qsh[D];
    __shared__ float part[256];
    __shared__ float ssh[128];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int64_t row = blockIdx.x;
    const int b = (int)(row / p.Hq);
    constexpr int m = M;
    const bool sketch = M > 0 && !p.s_ident;
    // loads: this thread's S^T entries, then (wave 0) the query
    const int l = t % (M > 0 ? M : 1), prt = t / (M > 0 ? M : 1);
    float sk[NI];
    if (sketch) {
#pragma unroll
        for (int k = 0; k < NI; ++k) sk[k] = p.sketch_t[(int64_t)(prt * NI + k) * M + l];
    }
    float x[VPL];
    int shq = 0;
    if (wave == 0) {
        float sg[VPL];
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const int64_t e = row * D + lane + 64 * v;
            x[v] = p.bf16 ? __uint_as_float((uint32_t) static_cast<const uint16_t*>(p.q)[e] << 16)
                          : static_cast<const float*>(p.q)[e];
            sg[v] = p.norot ? 1.0f : p.sigma[lane + 64 * v];
        }
        if (p.rope_cos) {
            const int pos = dev::query_pos(p.q_pos, p.seq_len, b, p.L_cap);
            const float c = p.rope_cos[(int64_t)pos * (D / 2) + lane % (D / 2)];
            const float sn = p.rope_sin[(int64_t)pos * (D / 2) + lane % (D / 2)];
            // RoPE: pair (i, i + d/2) in one lane (d = 128) or lanes l, l ^ 32 (d = 64)
            if constexpr (VPL == 2) {
                const float lo = x[0], hi = x[1];
                x[0] = lo * c - hi * sn;
                x[1] = hi * c + lo * sn;
            } else {
                const float own = x[0], other = __shfl_xor(own, 32);
                x[0] = lane < 32 ? own * c - other * sn : own * c + other * sn;
            }
        }
        if (!p.norot) {
#pragma unroll
            for (int v = 0; v < VPL; ++v) x[v] *= sg[v];
            // H_d in Sylvester order: butterflies over every index bit
#pragma unroll
            for (int sp = 1; sp < 64; sp <<= 1) {
#pragma unroll
                for (int v = 0; v < VPL; ++v) {
                    const float o = __shfl_xor(x[v], sp);
                    x[v] = (lane & sp) ? o - x[v] : x[v] + o;
                }
            }
            if constexpr (VPL == 2) {
                const float a0 = x[0], a1 = x[1];
                x[0] = a0 + a1;
                x[1] = a0 - a1;
            }
            const float inv = 1.0f / sqrtf((float)D);
#pragma unroll
            for (int v = 0; v < VPL; ++v) x[v] *= inv;
        }
        float amax = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) amax = fmaxf(amax, fabsf(x[v]));
        shq = fixed_shift(wave_max(amax));
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const int i = lane + 64 * v;
            qsh[i] = x[v];
            int8_t d[4];
            digits4(to_fixed(x[v], shq), d);
#pragma unroll
            for (int a = 0; a < 4; ++a) p.qd[(row * 4 + a) * D + i] = d[a];
        }
    }
    if constexpr (M == 0) {
        if (t == 0) {
            p.scale[row * 3 + 0] = (float)shq;
            p.scale[row * 3 + 1] = 0.0f;
            p.scale[row * 3 + 2] = 0.0f;
        }
        return;
    }
    __syncthreads();
    // partial sums of s = S q' (or s = q')
    if (sketch) {
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < NI; ++k) acc = fmaf(sk[k], qsh[prt * NI + k], acc);
        part[t] = acc;
    }
    __syncthreads();
    float sv = 0.0f;
    if (t < m) {
        if (sketch) {
            for (int k = 0; k < NT; ++k) sv += part[k * M + t];
        } else {
            sv = qsh[t];
        }
        ssh[t] = sv;
    }
    __syncthreads();
    if (wave == 0) {
        float smax = 0.0f;
        double sf = 0.0;
        for (int li = lane; li < m; li += 64) smax = fmaxf(smax, fabsf(ssh[li]));
        const int shs = fixed_shift(wave_max(smax));
        for (int li = lane; li < m; li += 64) sf += (double)to_fixed(ssh[li], shs);
        sf = wave_sum(sf);
        // sketch digits in MFMA slot order: byte (qk*ncs + cs)*16 + j holds
        // sketch row qk*(m/4) + 16*cs + j (zero where that slot is past m/4)
        for (int off = lane; off < p.sdw; off += 64) {
            const int qk = off / (16 * p.ncs), rem = off % (16 * p.ncs);
            const int cs = rem / 16, j = rem % 16;
            int8_t d[4] = {0, 0, 0, 0};
            if (16 * cs + j < m / 4) digits4(to_fixed(ssh[qk * (m / 4) + 16 * cs + j], shs), d);
#pragma unroll
            for (int a = 0; a < 4; ++a) p.sd[(row * 4 + a) * p.sdw + off] = d[a];
        }
        if (lane == 0) {
            p.scale[row * 3 + 0] = (float)shq;  // shifts are small integers, exact in fp32
            p.scale[row * 3 + 1] = (float)shs;
            p.scale[row * 3 + 2] = (float)ldexp(sf, -shs);
        }
    }
}

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// the integer-digit tile of the fused decode serves the fused scan's codebooks
bool logits_mfma_supported(const tq_codebook* ck) { return scan_supported(ck); }

size_t qdigits_workspace_bytes(const tq_codebook* ck, int64_t rows) {
    const size_t d = ck->spec.d, m = ck->spec.m;
    const size_t ncs = m == 0 ? 0 : std::max<size_t>(1, m / 64);
    const size_t sdw = 64 * ncs;
    return al256(rows * d * 4) + al256(rows * (m ? m : 1) * 4) + al256(rows * 4 * d) + al256(rows * 4 * (sdw ? sdw : 1)) +
           al256(rows * 3 * 4);
}

QDigits carve_qdigits(const tq_codebook* ck, void* ws, int64_t rows) {
    const size_t d = ck->spec.d, m = ck->spec.m;
    const size_t ncs = m == 0 ? 0 : std::max<size_t>(1, m / 64);
    const size_t sdw = 64 * ncs;
    char* p = static_cast<char*>(ws);
    QDigits q;
    q.qp = reinterpret_cast<float*>(p);
    p += al256(rows * d * 4);
    q.s = reinterpret_cast<float*>(p);
    p += al256(rows * (m ? m : 1) * 4);
    q.qd = reinterpret_cast<int8_t*>(p);
    p += al256(rows * 4 * d);
    q.sd = reinterpret_cast<int8_t*>(p);
    p += al256(rows * 4 * (sdw ? sdw : 1));
    q.scale = reinterpret_cast<float*>(p);
    q.sdw = (int)sdw;
    q.ncs = (int)ncs;
    return q;
}

hipError_t launch_qdigits(const tq_codebook* ck, const AttnArgs& a, const QDigits& q, hipStream_t stream) {
    QDig p{};
    p.q = a.q;
    p.bf16 = a.bf16;
    p.Hq = a.Hq;
    p.L_cap = a.L_cap;
    p.m = ck->spec.m;
    p.sdw = q.sdw;
    p.ncs = q.ncs;
    p.rows = (int64_t)a.B * a.Hq;
    p.seq_len = a.seq_len;
    p.q_pos = a.q_pos;
    p.rope_cos = a.rope_cos;
    p.rope_sin = a.rope_sin;
    p.sigma = ck->dev.sigma;
    p.sketch_t = ck->dev.sketch_t;
    p.norot = no_rotation(ck) ? 1 : 0;
    p.s_ident = sign_corr(ck) ? 1 : 0;
    p.qd = q.qd;
    p.sd = q.sd;
    p.scale = q.scale;
    const unsigned grid = (unsigned)p.rows;
    if (grid == 0) return hipSuccess;
    using Fn = void (*)(QDig);
    Fn fn = nullptr;
    const bool d64 = ck->spec.d == 64;
    switch (p.m) {
        case 0: fn = d64 ? qprep_digits_kernel<64, 0> : qprep_digits_kernel<128, 0>; break;
        case 32: fn = d64 ? qprep_digits_kernel<64, 32> : qprep_digits_kernel<128, 32>; break;
        case 64: fn = d64 ? qprep_digits_kernel<64, 64> : qprep_digits_kernel<128, 64>; break;
        case 128: fn = d64 ? qprep_digits_kernel<64, 128> : qprep_digits_kernel<128, 128>; break;
    }
    if (!fn) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace tq
