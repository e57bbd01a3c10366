// Decode-side kernels: attention logits from packed keys and the fused
// decode (softmax times values) from packed keys and values.
//
// Estimator (iaemfoco post, "TurboQuant: Uma Nova Abordagem"; itstec post,
// "Por dentro do processo de compressao KV"; tambur post for logits straight
// from quantised keys): with q' = Pi RoPE(q) and s = S q',
//     logit = nu ( <q', t[c]> + sqrt(pi/2)/m * gamma * <s, z> ),  z in {-1,+1}^m.
// Fused decode (TurboESM summary, technical section 2: dequantisation,
// residual correction and online softmax in one kernel, no dequantised copy
// of the cache): each workgroup owns a split of the key axis for one group
// of queries sharing a KV head, keeps a running max and sum, and accumulates
// p nu_v t[c_v] (d values, rotated domain) and p nu_v gamma_v z_v (m values,
// sketch domain).  A merge kernel combines the splits by log-sum-exp and
// returns to the original domain once per query:
//     out = Pi_v^T (A_y + sqrt(pi/2)/m_v S_v^T A_z) / l
// (FibQuant summary, section 2.3: lookup, inverse rotation, norm scale).
//
// Work layout: Hadamard codebooks (d = 64, 128) use one thread per key for
// the logit (codes unpacked in registers, the queries' q' and s broadcast
// from LDS, GT queries per pass) and, in the decode kernel, one thread per
// output coordinate for the value accumulation over keys staged in LDS.
// Dense (Haar) codebooks score by an MFMA GEMM over a dequantised chunk.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr float kQjl = 1.2533141373155003f;  // sqrt(pi / 2)
constexpr int kTopKMax = 16;

__device__ __forceinline__ float load_q(const void* q, int bf16, int64_t i) {
    if (bf16) return __uint_as_float((uint32_t) static_cast<const uint16_t*>(q)[i] << 16);
    return static_cast<const float*>(q)[i];
}

__device__ __forceinline__ int clamp_len(const int32_t* seq_len, int b, int L_cap) {
    int s = seq_len[b];
    return s < 0 ? 0 : (s > L_cap ? L_cap : s);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// ------------------------------------------------------------ query prep
struct QPrep {
    const void* q;
    int32_t bf16, Hq, L_cap, d, m;
    const int32_t* seq_len;
    const int32_t* q_pos;
    const float* rope_cos;
    const float* rope_sin;
    const float* sigma;
    const float* sketch;
    float* qp;  // [B*Hq][d]
    float* s;   // [B*Hq][m]
};

// q' = H (sigma * RoPE(q)) / sqrt(d), s = S q'; one workgroup per query head
template <int D>
__global__ __launch_bounds__(256) void qprep_rht_kernel(QPrep p) {
    __shared__ float xs[D];
    const int t = threadIdx.x;
    const int64_t bh = blockIdx.x;
    const int b = (int)(bh / p.Hq);
    if (t < D) xs[t] = load_q(p.q, p.bf16, bh * D + t);
    __syncthreads();
    if (p.rope_cos) {
        const int pos = dev::query_pos(p.q_pos, p.seq_len, b, p.L_cap);
        float lo = 0.f, hi = 0.f;
        if (t < D / 2) {
            const float c = p.rope_cos[(int64_t)pos * (D / 2) + t];
            const float sn = p.rope_sin[(int64_t)pos * (D / 2) + t];
            const float a = xs[t], bb = xs[t + D / 2];
            lo = a * c - bb * sn;
            hi = bb * c + a * sn;
        }
        __syncthreads();
        if (t < D / 2) {
            xs[t] = lo;
            xs[t + D / 2] = hi;
        }
        __syncthreads();
    }
    if (t < D) xs[t] *= p.sigma[t];
    __syncthreads();
    for (int s = 1; s < D; s <<= 1) {
        if (t < D / 2) {
            const int i = (t / s) * 2 * s + (t % s);
            const float a = xs[i], bb = xs[i + s];
            xs[i] = a + bb;
            xs[i + s] = a - bb;
        }
        __syncthreads();
    }
    const float inv = 1.0f / sqrtf((float)D);
    if (t < D) {
        xs[t] *= inv;
        p.qp[bh * D + t] = xs[t];
    }
    __syncthreads();
    for (int l = t; l < p.m; l += blockDim.x) {
        const float* row = p.sketch + (int64_t)l * D;
        float acc = 0.f;
        for (int i = 0; i < D; ++i) acc = fmaf(row[i], xs[i], acc);
        p.s[bh * p.m + l] = acc;
    }
}

// RoPE'd query rows (fp32) for the dense path: out[bh][d]
__global__ __launch_bounds__(256) void qrope_kernel(QPrep p, float* out) {
    const int64_t bh = blockIdx.x;
    const int b = (int)(bh / p.Hq);
    const int half = p.d / 2;
    for (int i = threadIdx.x; i < half; i += blockDim.x) {
        float a = load_q(p.q, p.bf16, bh * p.d + i);
        float bb = load_q(p.q, p.bf16, bh * p.d + i + half);
        if (p.rope_cos) {
            const int pos = dev::query_pos(p.q_pos, p.seq_len, b, p.L_cap);
            const float c = p.rope_cos[(int64_t)pos * half + i];
            const float sn = p.rope_sin[(int64_t)pos * half + i];
            const float a2 = a * c - bb * sn;
            const float b2 = bb * c + a * sn;
            a = a2;
            bb = b2;
        }
        out[bh * p.d + i] = a;
        out[bh * p.d + i + half] = bb;
    }
}

// -------------------------------------------------------- logit scan (RHT)
struct LogK {
    const float* qp;
    const float* s;
    const float* levels;
    const float* norm;
    const float* rnorm;
    const uint32_t* codes;
    const uint32_t* signs;
    const int32_t* seq_len;
    int32_t Hq, h_kv, L_cap, m, ngroups;
    int32_t k0, klen;   // keys [k0, k0 + klen) of each (b, kh)
    float* out;         // row (b*Hq + head), column (key - col0)
    int64_t ld;
    int32_t col0;
};

template <int D, int BITS>
__device__ __forceinline__ uint32_t code_at(const uint32_t* cw, int i) {
    return dev::code_get(cw, dev::code_loc(i, BITS), BITS);
}

template <int D, int BITS, int GT>
__global__ __launch_bounds__(256) void logits_rht_kernel(LogK p) {
    constexpr int CW = BITS * D / 32;
    __shared__ float qs[GT * D];
    __shared__ float ss[GT * D];  // m <= d for Hadamard codebooks
    __shared__ float lvl[16];
    const int t = threadIdx.x;
    const int grp = blockIdx.x % p.ngroups;
    const int64_t bk = blockIdx.x / p.ngroups;
    const int b = (int)(bk / p.h_kv);
    const int kh = (int)(bk % p.h_kv);
    const int G = p.Hq / p.h_kv;
    const int g0 = grp * GT;
    for (int idx = t; idx < GT * D; idx += 256) {
        const int g = idx / D, i = idx % D;
        const int64_t row = (int64_t)b * p.Hq + kh * G + g0 + g;
        qs[idx] = (g0 + g < G) ? p.qp[row * D + i] : 0.f;
    }
    for (int idx = t; idx < GT * p.m; idx += 256) {
        const int g = idx / p.m, l = idx % p.m;
        const int64_t row = (int64_t)b * p.Hq + kh * G + g0 + g;
        ss[g * D + l] = (g0 + g < G) ? p.s[row * p.m + l] : 0.f;
    }
    if (t < 16) lvl[t] = p.levels[t];
    __syncthreads();
    const int sl = clamp_len(p.seq_len, b, p.L_cap);
    const int j = p.k0 + blockIdx.y * 256 + t;
    if (j >= sl || j >= p.k0 + p.klen) return;
    const int64_t n = bk * p.L_cap + j;
    uint32_t cw[CW];
    const uint32_t* src = p.codes + n * CW;
#pragma unroll
    for (int w = 0; w < CW; ++w) cw[w] = src[w];
    float acc[GT];
#pragma unroll
    for (int g = 0; g < GT; ++g) acc[g] = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) {
        const float y = lvl[code_at<D, BITS>(cw, i)];
#pragma unroll
        for (int g = 0; g < GT; ++g) acc[g] = fmaf(qs[g * D + i], y, acc[g]);
    }
    float accs[GT];
#pragma unroll
    for (int g = 0; g < GT; ++g) accs[g] = 0.f;
    const int mw = p.m >> 5;
    for (int w = 0; w < mw; ++w) {
        const uint32_t word = p.signs[n * mw + w];
#pragma unroll
        for (int bit = 0; bit < 32; ++bit) {
            const float z = ((word >> bit) & 1u) ? 1.0f : -1.0f;
#pragma unroll
            for (int g = 0; g < GT; ++g) accs[g] = fmaf(ss[g * D + w * 32 + bit], z, accs[g]);
        }
    }
    const float nu = p.norm[n];
    const float cg = p.m ? (kQjl / (float)p.m) * p.rnorm[n] : 0.f;
#pragma unroll
    for (int g = 0; g < GT; ++g) {
        if (g0 + g < G) {
            const int64_t row = (int64_t)b * p.Hq + kh * G + g0 + g;
            p.out[row * p.ld + (j - p.col0)] = nu * (acc[g] + cg * accs[g]);
        }
    }
}

// ----------------------------------------------------------------- top-k
struct TopK {
    const float* scores;  // [rows][ld] relative to row0, column c holds key col0 + c
    int64_t ld;
    int64_t row0;         // absolute row (b*Hq + head) of workgroup 0
    int32_t col0, cnt;    // keys [col0, col0 + cnt)
    int32_t Hq, L_cap, k, first;
    const int32_t* seq_len;
    float* out_val;       // [rows][k]
    int32_t* out_idx;
};

__device__ __forceinline__ bool better(float a, int ia, float b, int ib) {
    return a > b || (a == b && ia < ib);
}

// One workgroup per row.  Each wave keeps its best k in lanes 0..k-1 (sorted
// by `better`) and the k-th as a threshold: a batch of 64 scores costs one
// compare and a ballot, and only the few that beat the threshold are
// inserted, one at a time (a shift of the lanes behind the insertion
// point).  Wave 0 then takes in the other waves' lists, and the running list
// of earlier chunks first.
__global__ __launch_bounds__(256) void topk_merge_kernel(TopK p) {
    __shared__ float lv[4][kTopKMax];
    __shared__ int li[4][kTopKMax];
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int64_t rel = blockIdx.x;
    const int64_t row = p.row0 + rel;
    const int b = (int)(row / p.Hq);
    const int sl = clamp_len(p.seq_len, b, p.L_cap);
    const int k = p.k;
    float kv = -INFINITY, thv = -INFINITY;
    int ki = 0x7fffffff, thi = 0x7fffffff;
    // every lane offers (x, id) when `valid`; NaN is never kept
    auto offer = [&](float x, int id, bool valid) {
        unsigned long long mask = __ballot(valid && x == x && better(x, id, thv, thi));
        while (mask) {
            const int l = __ffsll(mask) - 1;
            mask &= mask - 1;
            const float cv = __shfl(x, l);
            const int ci = __shfl(id, l);
            if (!better(cv, ci, thv, thi)) continue;  // the threshold rose meanwhile
            const int pos = __popcll(__ballot(lane < k && better(kv, ki, cv, ci)));
            const float uv = __shfl_up(kv, 1);
            const int ui = __shfl_up(ki, 1);
            if (lane < k && lane > pos) {
                kv = uv;
                ki = ui;
            }
            if (lane == pos) {
                kv = cv;
                ki = ci;
            }
            thv = __shfl(kv, k - 1);
            thi = __shfl(ki, k - 1);
        }
    };
    if (wave == 0 && !p.first) {
        const int id = lane < k ? p.out_idx[row * k + lane] : -1;
        offer(lane < k ? p.out_val[row * k + lane] : -INFINITY, id, lane < k && id >= 0);
    }
    const int hi = min(p.col0 + p.cnt, sl);
    for (int key0 = p.col0 + 64 * wave; key0 < hi; key0 += 256) {  // the same for the whole wave
        const int key = key0 + lane;
        const bool ok = key < hi;
        offer(ok ? p.scores[rel * p.ld + (key - p.col0)] : -INFINITY, key, ok);
    }
    if (lane < k) {
        lv[wave][lane] = kv;
        li[wave][lane] = ki;
    }
    __syncthreads();
    if (wave != 0) return;
    for (int w = 1; w < 4; ++w) {
        const float x = lane < k ? lv[w][lane] : -INFINITY;
        const int id = lane < k ? li[w][lane] : 0x7fffffff;
        offer(x, id, lane < k && id != 0x7fffffff);
    }
    if (lane < k) {
        const bool ok = ki != 0x7fffffff;
        p.out_val[row * k + lane] = ok ? kv : -INFINITY;
        p.out_idx[row * k + lane] = ok ? ki : -1;
    }
}

// ------------------------------------------------- dense (Haar) scoring
struct DenseScan {
    const float* levels;
    const float* norm;
    const float* rnorm;
    const uint32_t* codes;
    const uint32_t* signs;
    int32_t d, m, bits;
    int32_t block;  // vector codebooks: levels holds the N x block codewords
    int64_t rec0;   // record index of key 0 of this (b, kh)
    int32_t k0, cnt;
    float* aug;     // [cnt][d + m]: t[c], then sqrt(pi/2)/m gamma z
};

// vector codebooks: aug[r] = the concatenated codewords of key k0 + r (the
// rotated unit vector's estimate; FibQuant summary, section 2.3)
__global__ __launch_bounds__(256) void dense_vq_dequant_kernel(DenseScan p) {
    const int k = p.block, nb = p.d / k;
    const int cw = (p.bits * nb + 31) / 32;
    const uint32_t mask = (1u << p.bits) - 1u;
    for (int64_t r = blockIdx.x; r < p.cnt; r += gridDim.x) {
        const int64_t n = p.rec0 + p.k0 + r;
        const uint32_t* c = p.codes + n * cw;
        float* dst = p.aug + r * p.d;
        for (int j = threadIdx.x; j < nb; j += blockDim.x) {
            const int o = j * p.bits;
            uint32_t idx = c[o >> 5] >> (o & 31);
            if ((o & 31) + p.bits > 32) idx |= c[(o >> 5) + 1] << (32 - (o & 31));
            idx &= mask;
            for (int i = 0; i < k; ++i) dst[j * k + i] = p.levels[idx * k + i];
        }
    }
}

__global__ __launch_bounds__(256) void dense_dequant_kernel(DenseScan p) {
    const int width = p.d + p.m;
    const int cw = p.bits * p.d / 32, mw = p.m / 32;
    const uint32_t mask = (1u << p.bits) - 1u;
    const float cq = p.m ? kQjl / (float)p.m : 0.f;
    for (int64_t r = blockIdx.x; r < p.cnt; r += gridDim.x) {
        const int64_t n = p.rec0 + p.k0 + r;
        const uint32_t* c = p.codes + n * cw;
        float* dst = p.aug + r * width;
        for (int i = threadIdx.x; i < p.d; i += blockDim.x)
            dst[i] = p.levels[dev::code_get(c, dev::code_loc(i, p.bits), p.bits) & mask];
        if (p.m) {
            const float g = cq * p.rnorm[n];
            const uint32_t* sg = p.signs + n * mw;
            for (int l = threadIdx.x; l < p.m; l += blockDim.x)
                dst[p.d + l] = ((sg[l >> 5] >> (l & 31)) & 1u) ? g : -g;
        }
    }
}

// scores[g][c] *= nu of key k0 + c for keys below seq_len; with `out`
// given, those scores are also copied to out[g][k0 + c] (row stride out_ld)
__global__ __launch_bounds__(256) void finalize_scores_kernel(float* scores, int64_t ld, int rows, int cnt,
                                                              const float* norm, int64_t rec0, int k0,
                                                              const int32_t* seq_len, int b, int L_cap,
                                                              float* out, int64_t out_ld) {
    const int sl = clamp_len(seq_len, b, L_cap);
    const int64_t total = (int64_t)rows * cnt;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t g = e / cnt;
        const int c = (int)(e % cnt);
        if (k0 + c >= sl) continue;
        const float v = scores[g * ld + c] * norm[rec0 + k0 + c];
        scores[g * ld + c] = v;
        if (out) out[g * out_ld + k0 + c] = v;
    }
}

// ------------------------------------------------------------- decode
struct DecK {
    const float* qp;
    const float* s;
    const float* lv_k;
    const float* lv_v;
    const float* k_norm;
    const float* k_rnorm;
    const uint32_t* k_codes;
    const uint32_t* k_signs;
    const float* v_norm;
    const float* v_rnorm;
    const uint32_t* v_codes;
    const uint32_t* v_signs;
    const int32_t* seq_len;
    int32_t Hq, h_kv, L_cap, m, ngroups, nsplit, chunk;
    float scale;
    float* part;  // [B*Hq][nsplit][2 + d + m]
};

template <int D, int BITS, int GT>
__global__ __launch_bounds__(256) void decode_split_kernel(DecK p) {
    constexpr int CW = BITS * D / 32;
    extern __shared__ float lds[];
    const int m = p.m, mw = m >> 5;
    float* qs = lds;                      // [GT][D]
    float* ss = qs + GT * D;              // [GT][D]   (m <= D)
    float* lvk = ss + GT * D;             // [16]
    float* lvv = lvk + 16;                // [16]
    float* pv = lvv + 16;                 // [256][GT]  p * nu_v
    float* pz = pv + 256 * GT;            // [256][GT]  p * nu_v * gamma_v
    float* red = pz + 256 * GT;           // [4][GT]
    float* mrun = red + 4 * GT;           // [GT]
    float* lrun = mrun + GT;              // [GT]
    float* alpha = lrun + GT;             // [GT]
    uint32_t* vc = reinterpret_cast<uint32_t*>(alpha + GT);  // [256][CW]
    uint32_t* vs = vc + 256 * CW;                            // [256][mw]

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int grp = blockIdx.x % p.ngroups;
    const int64_t bk = blockIdx.x / p.ngroups;
    const int b = (int)(bk / p.h_kv);
    const int kh = (int)(bk % p.h_kv);
    const int G = p.Hq / p.h_kv;
    const int g0 = grp * GT;
    const int split = blockIdx.y;
    for (int idx = t; idx < GT * D; idx += 256) {
        const int g = idx / D, i = idx % D;
        const int64_t row = (int64_t)b * p.Hq + kh * G + g0 + g;
        qs[idx] = (g0 + g < G) ? p.qp[row * D + i] : 0.f;
        ss[idx] = (g0 + g < G && i < m) ? p.s[row * m + i] : 0.f;
    }
    if (t < 16) {
        lvk[t] = p.lv_k[t];
        lvv[t] = p.lv_v[t];
    }
    if (t < GT) {
        mrun[t] = -INFINITY;
        lrun[t] = 0.f;
    }
    __syncthreads();

    const int sl = clamp_len(p.seq_len, b, p.L_cap);
    const int c0 = split * p.chunk;
    const int c1 = min(c0 + p.chunk, sl);
    const float cqk = m ? kQjl / (float)m : 0.f;

    // coordinate role of this thread in the value accumulation
    const bool ycoord = t < D;
    const bool zcoord = !ycoord && t < D + m;
    const dev::CodeLoc cl = dev::code_loc(ycoord ? t : 0, BITS);
    const int zl = t - D;
    float acc[GT];
#pragma unroll
    for (int g = 0; g < GT; ++g) acc[g] = 0.f;

    for (int base = c0; base < c1; base += 256) {
        const int j = base + t;
        const bool valid = j < c1;
        const int64_t n = bk * p.L_cap + j;
        float a[GT];
        float nu_v = 0.f, gm_v = 0.f;
        if (valid) {
            uint32_t cw[CW];
            const uint32_t* src = p.k_codes + n * CW;
#pragma unroll
            for (int w = 0; w < CW; ++w) cw[w] = src[w];
            float ay[GT], az[GT];
#pragma unroll
            for (int g = 0; g < GT; ++g) ay[g] = az[g] = 0.f;
#pragma unroll
            for (int i = 0; i < D; ++i) {
                const float y = lvk[code_at<D, BITS>(cw, i)];
#pragma unroll
                for (int g = 0; g < GT; ++g) ay[g] = fmaf(qs[g * D + i], y, ay[g]);
            }
            for (int w = 0; w < mw; ++w) {
                const uint32_t word = p.k_signs[n * mw + w];
#pragma unroll
                for (int bit = 0; bit < 32; ++bit) {
                    const float z = ((word >> bit) & 1u) ? 1.0f : -1.0f;
#pragma unroll
                    for (int g = 0; g < GT; ++g) az[g] = fmaf(ss[g * D + w * 32 + bit], z, az[g]);
                }
            }
            const float nu = p.k_norm[n];
            const float cg = m ? cqk * p.k_rnorm[n] : 0.f;
#pragma unroll
            for (int g = 0; g < GT; ++g) a[g] = p.scale * (nu * (ay[g] + cg * az[g]));
            // stage the value record of key j
            const uint32_t* vsrc = p.v_codes + n * CW;
#pragma unroll
            for (int w = 0; w < CW; ++w) vc[t * CW + w] = vsrc[w];
            for (int w = 0; w < mw; ++w) vs[t * mw + w] = p.v_signs[n * mw + w];
            nu_v = p.v_norm[n];
            gm_v = m ? p.v_rnorm[n] : 0.f;
        } else {
#pragma unroll
            for (int g = 0; g < GT; ++g) a[g] = -INFINITY;
        }
        // block max of this sub-block, new running max and rescale factor
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            const float wm = wave_max(a[g]);
            if (lane == 0) red[wave * GT + g] = wm;
        }
        __syncthreads();
        if (t < GT) {
            const float bm = fmaxf(fmaxf(red[t], red[GT + t]), fmaxf(red[2 * GT + t], red[3 * GT + t]));
            const float mo = mrun[t];
            const float mn = fmaxf(mo, bm);
            alpha[t] = (mn == -INFINITY) ? 1.0f : expf(mo - mn);
            mrun[t] = mn;
        }
        __syncthreads();
        float psum[GT];
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            const float pj = valid ? expf(a[g] - mrun[g]) : 0.f;
            psum[g] = pj;
            pv[t * GT + g] = pj * nu_v;
            pz[t * GT + g] = pj * nu_v * gm_v;
        }
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            const float ws = wave_sum(psum[g]);
            if (lane == 0) red[wave * GT + g] = ws;
        }
        __syncthreads();
        if (t < GT) lrun[t] = lrun[t] * alpha[t] + (red[t] + red[GT + t] + red[2 * GT + t] + red[3 * GT + t]);
#pragma unroll
        for (int g = 0; g < GT; ++g) acc[g] *= alpha[g];
        const int cnt = min(256, c1 - base);
        if (ycoord) {
            for (int jj = 0; jj < cnt; ++jj) {
                const float y = lvv[dev::code_get(vc + jj * CW, cl, BITS)];
#pragma unroll
                for (int g = 0; g < GT; ++g) acc[g] = fmaf(pv[jj * GT + g], y, acc[g]);
            }
        } else if (zcoord) {
            for (int jj = 0; jj < cnt; ++jj) {
                const float z = ((vs[jj * mw + (zl >> 5)] >> (zl & 31)) & 1u) ? 1.0f : -1.0f;
#pragma unroll
                for (int g = 0; g < GT; ++g) acc[g] = fmaf(pz[jj * GT + g], z, acc[g]);
            }
        }
        __syncthreads();
    }
    const int width = 2 + D + m;
#pragma unroll
    for (int g = 0; g < GT; ++g) {
        if (g0 + g >= G) continue;
        const int64_t row = (int64_t)b * p.Hq + kh * G + g0 + g;
        float* dst = p.part + (row * p.nsplit + split) * width;
        if (t == 0) {
            dst[0] = mrun[g];
            dst[1] = lrun[g];
        }
        if (t < D + m) dst[2 + t] = acc[g];
    }
}

struct MergeK {
    const float* part;
    int32_t nsplit, d, m;
    const float* sigma;   // Hadamard form
    const float* sketch;  // [m][d]
    float corr;           // scale of the correction term (sqrt(pi/2)/m, or 1 for the sign correction)
    int32_t s_ident;      // S = I (sign correction): S^T A_z = A_z
    int32_t norot;        // Pi = I: no inverse rotation
    float* out;           // [B*Hq][d]
};

// log-sum-exp merge of the splits, then back to the original domain:
// out = sigma * H (A_y + sqrt(pi/2)/m S^T A_z) / (sqrt(d) l)
// The split maxima are read by all threads at once (one round trip), the
// column sums are unrolled so their loads are in flight together.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(MergeK p) {
    __shared__ float fw[256];  // exp(M_s - M) of the current batch of splits
    __shared__ float red[8];
    __shared__ float w[D];
    __shared__ float az[D];
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int64_t row = blockIdx.x;
    const int width = 2 + D + p.m;
    const float* base = p.part + row * p.nsplit * width;
    float mx = -INFINITY;
    for (int s = t; s < p.nsplit; s += 256) mx = fmaxf(mx, base[(int64_t)s * width]);
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float l = 0.f, acc = 0.f;
    const bool col = t < D + p.m;
    for (int s0 = 0; s0 < p.nsplit; s0 += 256) {
        const int cnt = min(256, p.nsplit - s0);
        float lw = 0.f;
        if (t < cnt) {
            const float ms = base[(int64_t)(s0 + t) * width];
            const float f = (ms == -INFINITY || mx == -INFINITY) ? 0.f : expf(ms - mx);
            fw[t] = f;
            lw = f * base[(int64_t)(s0 + t) * width + 1];
        }
        lw = wave_sum(lw);
        if (lane == 0) red[4 + wave] = lw;
        __syncthreads();
        l += (red[4] + red[5]) + (red[6] + red[7]);
        if (col) {
            const float* src = base + (int64_t)s0 * width + 2 + t;
            int s = 0;
            for (; s + 8 <= cnt; s += 8) {
                float v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = src[(int64_t)(s + u) * width];
#pragma unroll
                for (int u = 0; u < 8; ++u) acc = fmaf(fw[s + u], v[u], acc);
            }
            for (; s < cnt; ++s) acc = fmaf(fw[s], src[(int64_t)s * width], acc);
        }
        __syncthreads();
    }
    // (empty splits have weight 0 and all-zero columns, written by the split kernels)
    if (t >= D && col) az[t - D] = acc;
    __syncthreads();
    if (t < D) {
        float corr = 0.f;
        if (p.s_ident) {
            corr = p.m ? az[t] : 0.f;
        } else {
            // S^T A_z: sixteen sketch rows' loads in flight at a time (m is a multiple of 32)
            for (int k0 = 0; k0 < p.m; k0 += 16) {
                float sv[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) sv[u] = p.sketch[(int64_t)(k0 + u) * D + t];
#pragma unroll
                for (int u = 0; u < 16; ++u) corr = fmaf(sv[u], az[k0 + u], corr);
            }
        }
        w[t] = acc + p.corr * corr;
    }
    __syncthreads();
    if (p.norot) {
        if (t < D) p.out[row * D + t] = (l > 0.f) ? w[t] / l : 0.f;
        return;
    }
    for (int s = 1; s < D; s <<= 1) {
        if (t < D / 2) {
            const int i = (t / s) * 2 * s + (t % s);
            const float a = w[i], bb = w[i + s];
            w[i] = a + bb;
            w[i + s] = a - bb;
        }
        __syncthreads();
    }
    if (t < D) {
        const float o = (l > 0.f) ? p.sigma[t] * w[t] / (sqrtf((float)D) * l) : 0.f;
        p.out[row * D + t] = o;
    }
}

// The same merge for m in {0, 32, 64, 128}, arranged for latency (one
// workgroup per query row, few rows, so the loads' round trips dominate):
// every load that does not depend on another is issued at once - the
// thread's share of S (thread (kh, c) sums rows [kh m/(256/d), ...) of
// column c), the split maxima, and per 64 splits the thread's column of the
// partials - and the inverse Walsh-Hadamard transform runs in wave 0's
// registers (lane l holds coordinates l + 64 v) instead of through barriers.
template <int D, int M>
__global__ __launch_bounds__(256) void decode_merge_fast_kernel(MergeK p) {
    constexpr int VPL = D / 64;
    constexpr int KP = 256 / D;                  // threads per output column for S^T A_z
    constexpr int NK = M > 0 ? M / KP : 1;       // sketch rows per thread
    constexpr int W = 2 + D + M;
    __shared__ float fw[64];
    __shared__ float red[8];
    __shared__ float az[M > 0 ? M : 1];
    __shared__ float cpart[M > 0 ? 256 : 1];
    __shared__ float w[D];
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int64_t row = blockIdx.x;
    const float* base = p.part + row * p.nsplit * (int64_t)W;
    const bool col = t < D + M;
    const bool skt = M > 0 && !p.s_ident;
    // S rows of this thread's share (independent of everything else)
    float sk[NK];
    if (skt) {
        const int c = t % D, kh = t / D;
#pragma unroll
        for (int k = 0; k < NK; ++k) sk[k] = p.sketch[(int64_t)(kh * NK + k) * D + c];
    }
    // split maxima
    float mx = -INFINITY;
    for (int s = t; s < p.nsplit; s += 256) mx = fmaxf(mx, base[(int64_t)s * W]);
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float l = 0.0f, acc = 0.0f;
    for (int s0 = 0; s0 < p.nsplit; s0 += 64) {
        const int cnt = min(64, p.nsplit - s0);
        // the column's 64 partials (past the last split: a clamped reload, weight 0)
        float v[64];
        if (col) {
#pragma unroll
            for (int u = 0; u < 64; ++u) v[u] = base[(int64_t)min(s0 + u, p.nsplit - 1) * W + 2 + t];
        }
        __syncthreads();  // the previous chunk's weights have been used
        if (wave == 0) {
            const int64_t sr = (int64_t)min(s0 + lane, p.nsplit - 1) * W;
            const float ms = base[sr], ls = base[sr + 1];
            const float f = (lane >= cnt || ms == -INFINITY || mx == -INFINITY) ? 0.0f : expf(ms - mx);
            fw[lane] = f;
            const float lw = wave_sum(f * ls);
            if (lane == 0) red[4] = lw;
        }
        __syncthreads();
        l += red[4];
        if (col) {
#pragma unroll
            for (int u = 0; u < 64; ++u) acc = fmaf(fw[u], v[u], acc);
        }
    }
    // (empty splits have weight 0 and all-zero columns, written by the split kernels)
    if constexpr (M > 0) {
        if (t >= D && col) az[t - D] = acc;
        __syncthreads();
        if (skt) {
            const int kh = t / D;
            float cr = 0.0f;
#pragma unroll
            for (int k = 0; k < NK; ++k) cr = fmaf(sk[k], az[kh * NK + k], cr);
            cpart[t] = cr;
        }
        __syncthreads();
        if (t < D) {
            float corr = 0.0f;
            if (skt) {
#pragma unroll
                for (int kk = 0; kk < KP; ++kk) corr += cpart[kk * D + t];
            } else {
                corr = az[t];
            }
            acc += p.corr * corr;
        }
    }
    if (t < D) w[t] = acc;
    __syncthreads();
    if (wave != 0) return;
    float x[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) x[v] = w[lane + 64 * v];
    if (!p.norot) {
        // H_d in Sylvester order, then the sign flips and 1/sqrt(d)
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
#pragma unroll
        for (int v = 0; v < VPL; ++v) x[v] = (l > 0.0f) ? p.sigma[lane + 64 * v] * x[v] / (sqrtf((float)D) * l) : 0.0f;
    } else {
#pragma unroll
        for (int v = 0; v < VPL; ++v) x[v] = (l > 0.0f) ? x[v] / l : 0.0f;
    }
#pragma unroll
    for (int v = 0; v < VPL; ++v) p.out[row * D + lane + 64 * v] = x[v];
}

// First merge stage for many splits: workgroup (row, g) combines splits
// [32 g, 32 g + 32) of the row by log-sum-exp into one partial of the same
// form (max, sum, A_y, A_z), so the final merge reads few partials.  The
// launch gives a thread per column (up to 512), so every column's 32 loads
// are in flight at once.
constexpr int kMergeGroup = 32;
__global__ __launch_bounds__(512) void decode_merge_group_kernel(const float* part, int nsplit, int width,
                                                                 float* out, int ngroup) {
    __shared__ float fw[kMergeGroup];
    __shared__ float red[2];
    const int t = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int g = blockIdx.y;
    const int s0 = g * kMergeGroup, cnt = min(kMergeGroup, nsplit - s0);
    const float* base = part + (row * nsplit + s0) * (int64_t)width;
    if (t < 64) {
        const float ms = t < cnt ? base[(int64_t)t * width] : -INFINITY;
        const float mx = wave_max(ms);
        const float f = (ms == -INFINITY) ? 0.f : expf(ms - mx);
        if (t < kMergeGroup) fw[t] = f;
        const float lw = wave_sum(t < cnt ? f * base[(int64_t)t * width + 1] : 0.f);
        if (t == 0) {
            red[0] = mx;
            red[1] = lw;
        }
    }
    __syncthreads();
    float* dst = out + (row * ngroup + g) * (int64_t)width;
    for (int c = t; c < width; c += blockDim.x) {
        float v;
        if (c == 0) v = red[0];
        else if (c == 1) v = red[1];
        else {
            float x[kMergeGroup];
#pragma unroll
            for (int s = 0; s < kMergeGroup; ++s) x[s] = s < cnt ? base[(int64_t)s * width + c] : 0.f;
            v = 0.f;
#pragma unroll
            for (int s = 0; s < kMergeGroup; ++s) v = fmaf(s < cnt ? fw[s] : 0.f, x[s], v);
        }
        dst[c] = v;
    }
}

// ------------------------------------------------------------ dispatch
using LogFn = void (*)(LogK);
using DecFn = void (*)(DecK);

template <int D, int BITS>
LogFn pick_log_gt(int gt) {
    return gt == 8 ? logits_rht_kernel<D, BITS, 8> : logits_rht_kernel<D, BITS, 4>;
}
template <int D>
LogFn pick_log_bits(int bits, int gt) {
    switch (bits) {
        case 1: return pick_log_gt<D, 1>(gt);
        case 2: return pick_log_gt<D, 2>(gt);
        case 3: return pick_log_gt<D, 3>(gt);
        case 4: return pick_log_gt<D, 4>(gt);
    }
    return nullptr;
}
LogFn pick_logits(int d, int bits, int gt) {
    if (d == 64) return pick_log_bits<64>(bits, gt);
    if (d == 128) return pick_log_bits<128>(bits, gt);
    return nullptr;
}
template <int D, int BITS>
DecFn pick_dec_gt(int gt) {
    return gt == 8 ? decode_split_kernel<D, BITS, 8> : decode_split_kernel<D, BITS, 4>;
}
template <int D>
DecFn pick_dec_bits(int bits, int gt) {
    switch (bits) {
        case 1: return pick_dec_gt<D, 1>(gt);
        case 2: return pick_dec_gt<D, 2>(gt);
        case 3: return pick_dec_gt<D, 3>(gt);
        case 4: return pick_dec_gt<D, 4>(gt);
    }
    return nullptr;
}
DecFn pick_decode(int d, int bits, int gt) {
    if (d == 64) return pick_dec_bits<64>(bits, gt);
    if (d == 128) return pick_dec_bits<128>(bits, gt);
    return nullptr;
}

int group_tile(int G) { return G >= 8 ? 8 : 4; }

constexpr int kScanChunk = 65536;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int decode_nsplit(int64_t bkg, int L_cap) {
    int64_t want = (2048 + bkg - 1) / bkg;
    int64_t maxs = (L_cap + 255) / 256;
    if (want > maxs) want = maxs;
    if (want < 1) want = 1;
    return (int)want;
}

int decode_chunk(int L_cap, int nsplit) {
    int c = (L_cap + nsplit - 1) / nsplit;
    return ((c + 255) / 256) * 256;
}

QPrep make_qprep(const tq_codebook* ck, const AttnArgs& a, float* qp, float* s) {
    QPrep q{};
    q.q = a.q;
    q.bf16 = a.bf16;
    q.Hq = a.Hq;
    q.L_cap = a.L_cap;
    q.d = ck->spec.d;
    q.m = ck->spec.m;
    q.seq_len = a.seq_len;
    q.q_pos = a.q_pos;
    q.rope_cos = a.rope_cos;
    q.rope_sin = a.rope_sin;
    q.sigma = ck->dev.sigma;
    q.sketch = ck->dev.sketch;
    q.qp = qp;
    q.s = s;
    return q;
}

}  // namespace

hipError_t launch_qprep_rht(const tq_codebook* ck, const AttnArgs& a, float* qp, float* s,
                            hipStream_t stream) {
    QPrep q = make_qprep(ck, a, qp, s);
    const unsigned grid = (unsigned)((int64_t)a.B * a.Hq);
    if (ck->spec.d == 64) hipLaunchKernelGGL(qprep_rht_kernel<64>, dim3(grid), dim3(256), 0, stream, q);
    else if (ck->spec.d == 128) hipLaunchKernelGGL(qprep_rht_kernel<128>, dim3(grid), dim3(256), 0, stream, q);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

// merge the scores of keys [col0, col0 + cnt) (rows row0.. of `scores`, ld
// apart) into the running top-k of every query row
hipError_t launch_topk(const AttnArgs& a, const float* scores, int64_t ld, int64_t row0, int col0, int cnt,
                       bool first, hipStream_t stream) {
    TopK tk{};
    tk.scores = scores;
    tk.ld = ld;
    tk.row0 = row0;
    tk.col0 = col0;
    tk.cnt = cnt;
    tk.Hq = a.Hq;
    tk.L_cap = a.L_cap;
    tk.k = a.top_k;
    tk.first = first;
    tk.seq_len = a.seq_len;
    tk.out_val = a.out;
    tk.out_idx = a.topk_idx;
    hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)((int64_t)a.B * a.Hq)), dim3(256), 0, stream, tk);
    return hipGetLastError();
}

size_t logits_workspace_bytes(const tq_codebook* ck, int64_t B, int Hq, int h_kv, int L_cap, int top_k) {
    const size_t d = ck->spec.d, m = ck->spec.m;
    const size_t rows = (size_t)B * Hq;
    const size_t chunk = (size_t)std::min(L_cap, kScanChunk);
    if (ck->spec.block >= 2 && !ck->dense) {
        size_t bytes = align256(rows * d * 4);
        if (top_k) bytes += align256(rows * chunk * 4);
        return bytes;
    }
    if (!ck->dense) {
        // the scan prepares its queries in LDS (one row tile per KV head, or two without a sketch)
        const int G = h_kv > 0 ? Hq / h_kv : 1;
        size_t bytes = !scan_supported(ck)           ? align256(rows * (d + m) * 4)
                       : scan_prepares_queries(ck, G) ? 0
                                                  : align256(qdigits_workspace_bytes(ck, (int64_t)rows));
        if (top_k) bytes += align256(rows * chunk * 4);
        return bytes;
    }
    const int G = h_kv > 0 ? Hq / h_kv : 0;
    size_t bytes = align256(rows * d * 4) + align256(rows * (d + m) * 4);  // rope'd q, [q' | s]
    if (ck->spec.block < 2 && gemm_records_supported(d, m, ck->spec.bits))
        bytes += align256(gemm_records_split_bytes((int64_t)rows, d, m));  // [q' | s] in bf16 pieces
    else
        bytes += align256(chunk * (d + m) * 4);                            // dequantised keys
    bytes += align256((size_t)G * chunk * 4);                              // scores
    (void)top_k;
    return bytes;
}

size_t decode_workspace_bytes(const tq_codebook* ck, const tq_codebook* cv, int64_t B, int Hq, int h_kv,
                              int L_cap) {
    const size_t d = ck->spec.d, mk = ck->spec.m, mv = cv->spec.m;
    const size_t rows = (size_t)B * Hq;
    const int G = h_kv > 0 ? Hq / h_kv : 1;
    const int gt = group_tile(G);
    const int64_t bkg = (int64_t)B * h_kv * ((G + gt - 1) / gt);
    if (ck->spec.block >= 2) {
        // q', split partials (M, l, A_y) and the merge's first stage
        int nsplit = 1, split_len = 0;
        vq_attn_plan(L_cap, &nsplit, &split_len);
        const size_t ngroup = (size_t)(nsplit + kMergeGroup - 1) / kMergeGroup;
        return align256(rows * d * 4) + align256(rows * nsplit * (2 + d) * 4) + align256(rows * ngroup * (2 + d) * 4);
    }
    if (decode_mfma_supported(ck, cv)) {
        int nsplit = 1, split_len = 0;
        decode_mfma_plan(B, Hq, h_kv, L_cap, &nsplit, &split_len);
        const size_t ngroup = (size_t)(nsplit + kMergeGroup - 1) / kMergeGroup;
        return align256(qdigits_workspace_bytes(ck, (int64_t)rows)) + align256(rows * nsplit * (2 + d + mv) * 4) +
               align256(rows * ngroup * (2 + d + mv) * 4);
    }
    const int ns = decode_nsplit(bkg > 0 ? bkg : 1, L_cap);
    return align256(rows * (d + mk) * 4) + align256(rows * ns * (2 + d + mv) * 4);
}

hipError_t launch_logits(const tq_codebook* ck, const tq_packed& k, const AttnArgs& a, hipStream_t stream) {
    const int d = ck->spec.d, m = ck->spec.m, bits = ck->spec.bits;
    const int G = a.Hq / a.h_kv;
    const int64_t rows = (int64_t)a.B * a.Hq;
    char* ws = static_cast<char*>(a.ws);
    const int chunk = std::min(a.L_cap, kScanChunk);
    if (ck->spec.block >= 2 && !ck->dense) {
        // vector codebook: q' = Pi RoPE(q), then codeword lookups fused into the dot products
        if (!vq_supported(ck)) return hipErrorInvalidValue;
        float* qp = reinterpret_cast<float*>(ws);
        float* scores = reinterpret_cast<float*>(ws + align256((size_t)rows * d * 4));
        hipError_t e = launch_qprep_rht(ck, a, qp, nullptr, stream);
        if (e != hipSuccess) return e;
        if (a.top_k == 0) return launch_vq_logits(ck, k, a, qp, 0, a.L_cap, a.out, a.L_cap, 0, stream);
        for (int k0 = 0; k0 < a.L_cap; k0 += chunk) {
            const int cnt = std::min(chunk, a.L_cap - k0);
            e = launch_vq_logits(ck, k, a, qp, k0, cnt, scores, chunk, k0, stream);
            if (e != hipSuccess) return e;
            e = launch_topk(a, scores, chunk, 0, k0, cnt, k0 == 0, stream);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    if (!ck->dense && scan_supported(ck)) {
        const bool fused = scan_prepares_queries(ck, G);
        QDigits qd{};
        char* wsc = ws;
        if (!fused) {
            qd = carve_qdigits(ck, ws, rows);
            wsc = ws + align256(qdigits_workspace_bytes(ck, rows));
            const hipError_t e = launch_qdigits(ck, a, qd, stream);
            if (e != hipSuccess) return e;
        }
        const QDigits* qp = fused ? nullptr : &qd;
        float* scores = reinterpret_cast<float*>(wsc);
        if (a.top_k == 0) return launch_scan(ck, k, a, qp, 0, a.L_cap, a.out, a.L_cap, 0, stream);
        for (int k0 = 0; k0 < a.L_cap; k0 += chunk) {
            const int cnt = std::min(chunk, a.L_cap - k0);
            hipError_t e = launch_scan(ck, k, a, qp, k0, cnt, scores, chunk, k0, stream);
            if (e != hipSuccess) return e;
            TopK tk{};
            tk.scores = scores;
            tk.ld = chunk;
            tk.row0 = 0;
            tk.col0 = k0;
            tk.cnt = cnt;
            tk.Hq = a.Hq;
            tk.L_cap = a.L_cap;
            tk.k = a.top_k;
            tk.first = k0 == 0;
            tk.seq_len = a.seq_len;
            tk.out_val = a.out;
            tk.out_idx = a.topk_idx;
            hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)rows), dim3(256), 0, stream, tk);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    if (!ck->dense) {
        float* qp = reinterpret_cast<float*>(ws);
        float* s = qp + rows * d;
        float* scores = reinterpret_cast<float*>(ws + align256(rows * (d + m) * 4));
        hipError_t e = launch_qprep_rht(ck, a, qp, s, stream);
        if (e != hipSuccess) return e;
        const int gt = group_tile(G);
        LogFn fn = pick_logits(d, bits, gt);
        if (!fn) return hipErrorInvalidValue;
        LogK p{};
        p.qp = qp;
        p.s = s;
        p.levels = ck->dev.levels;
        p.norm = k.norm;
        p.rnorm = k.rnorm;
        p.codes = k.codes;
        p.signs = k.signs;
        p.seq_len = a.seq_len;
        p.Hq = a.Hq;
        p.h_kv = a.h_kv;
        p.L_cap = a.L_cap;
        p.m = m;
        p.ngroups = (G + gt - 1) / gt;
        const unsigned gx = (unsigned)((int64_t)a.B * a.h_kv * p.ngroups);
        if (a.top_k == 0) {
            p.k0 = 0;
            p.klen = a.L_cap;
            p.out = a.out;
            p.ld = a.L_cap;
            p.col0 = 0;
            hipLaunchKernelGGL(fn, dim3(gx, (a.L_cap + 255) / 256), dim3(256), 0, stream, p);
            return hipGetLastError();
        }
        for (int k0 = 0; k0 < a.L_cap; k0 += chunk) {
            const int cnt = std::min(chunk, a.L_cap - k0);
            p.k0 = k0;
            p.klen = cnt;
            p.out = scores;
            p.ld = chunk;
            p.col0 = k0;
            hipLaunchKernelGGL(fn, dim3(gx, (cnt + 255) / 256), dim3(256), 0, stream, p);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
            TopK tk{};
            tk.scores = scores;
            tk.ld = chunk;
            tk.col0 = k0;
            tk.cnt = cnt;
            tk.Hq = a.Hq;
            tk.L_cap = a.L_cap;
            tk.k = a.top_k;
            tk.first = k0 == 0;
            tk.seq_len = a.seq_len;
            tk.out_val = a.out;
            tk.out_idx = a.topk_idx;
            hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)rows), dim3(256), 0, stream, tk);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    // dense rotation: q' and s by GEMM, keys dequantised per chunk (or formed inside the score GEMM), scores by GEMM
    float* qr = reinterpret_cast<float*>(ws);
    float* qaug = reinterpret_cast<float*>(ws + align256(rows * d * 4));
    float* aug = reinterpret_cast<float*>(ws + align256(rows * d * 4) + align256(rows * (d + m) * 4));
    // scalar codes of 1, 2 or 4 bits: [q' | s] split once into bf16 pieces
    // (in the dequantisation buffer's place) for the record-forming score GEMM
    const bool records = ck->spec.block < 2 && gemm_records_supported(d, m, bits);
    const size_t aug_bytes = records ? gemm_records_split_bytes((int64_t)rows, d, m) : (size_t)chunk * (d + m) * 4;
    float* scores = reinterpret_cast<float*>(ws + align256(rows * d * 4) + align256(rows * (d + m) * 4) +
                                             align256(aug_bytes));
    QPrep q = make_qprep(ck, a, nullptr, nullptr);
    hipLaunchKernelGGL(qrope_kernel, dim3((unsigned)rows), dim3(256), 0, stream, q, qr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_gemm_nt(qr, d, ck->dev.rot, d, qaug, d + m, (int)rows, d, d, stream);
    if (e != hipSuccess) return e;
    if (m) {
        e = launch_gemm_nt(qaug, d + m, ck->dev.sketch, d, qaug + d, d + m, (int)rows, m, d, stream);
        if (e != hipSuccess) return e;
    }
    if (records) {
        e = launch_split_rows(qaug, d + m, (int)rows, d + m, aug, stream);
        if (e != hipSuccess) return e;
    }
    for (int b = 0; b < a.B; ++b)
        for (int kh = 0; kh < a.h_kv; ++kh) {
            const int64_t rec0 = ((int64_t)b * a.h_kv + kh) * a.L_cap;
            const int64_t row0 = (int64_t)b * a.Hq + (int64_t)kh * G;
            for (int k0 = 0; k0 < a.L_cap; k0 += chunk) {
                const int cnt = std::min(chunk, a.L_cap - k0);
                DenseScan ds{};
                ds.levels = ck->dev.levels;
                ds.norm = k.norm;
                ds.rnorm = k.rnorm;
                ds.codes = k.codes;
                ds.signs = k.signs;
                ds.d = d;
                ds.m = m;
                ds.bits = bits;
                ds.block = ck->spec.block;
                ds.rec0 = rec0;
                ds.k0 = k0;
                ds.cnt = cnt;
                ds.aug = aug;
                if (records) {
                    // the score GEMM forms the keys' estimates from their records while it loads them
                    const RecB rb{k.codes, k.signs, k.rnorm, ck->dev.levels, rec0 + k0, d, m, bits};
                    e = launch_gemm_records(reinterpret_cast<const uint16_t*>(aug) + row0 * (d + m),
                                            (int64_t)rows * (d + m), G, rb, scores, chunk, cnt, stream);
                    if (e != hipSuccess) return e;
                } else {
                    if (ck->spec.block >= 2)
                        hipLaunchKernelGGL(dense_vq_dequant_kernel, dim3((unsigned)std::min(cnt, 8192)), dim3(256), 0,
                                           stream, ds);
                    else
                        hipLaunchKernelGGL(dense_dequant_kernel, dim3((unsigned)std::min(cnt, 8192)), dim3(256), 0,
                                           stream, ds);
                    e = hipGetLastError();
                    if (e != hipSuccess) return e;
                    e = launch_gemm_nt(qaug + row0 * (d + m), d + m, aug, d + m, scores, chunk, G, cnt, d + m, stream);
                    if (e != hipSuccess) return e;
                }
                const int64_t tot = (int64_t)G * cnt;
                const unsigned sg = (unsigned)std::min<int64_t>((tot + 255) / 256, 65536);
                hipLaunchKernelGGL(finalize_scores_kernel, dim3(sg), dim3(256), 0, stream, scores, (int64_t)chunk, G,
                                   cnt, k.norm, rec0, k0, a.seq_len, b, a.L_cap,
                                   a.top_k ? nullptr : a.out + row0 * a.L_cap, (int64_t)a.L_cap);
                e = hipGetLastError();
                if (e != hipSuccess) return e;
                if (a.top_k) {
                    TopK tk{};
                    tk.scores = scores;
                    tk.ld = chunk;
                    tk.col0 = k0;
                    tk.cnt = cnt;
                    tk.Hq = a.Hq;
                    tk.L_cap = a.L_cap;
                    tk.k = a.top_k;
                    tk.first = k0 == 0;
                    tk.seq_len = a.seq_len;
                    tk.row0 = row0;
                    tk.out_val = a.out;
                    tk.out_idx = a.topk_idx;
                    hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)G), dim3(256), 0, stream, tk);
                    e = hipGetLastError();
                    if (e != hipSuccess) return e;
                }
            }
        }
    return hipSuccess;
}

hipError_t launch_decode(const tq_codebook* ck, const tq_codebook* cv, const tq_packed& k, const tq_packed& v,
                         const AttnArgs& a, hipStream_t stream) {
    const int d = ck->spec.d, m = ck->spec.m, bits = ck->spec.bits;
    const int G = a.Hq / a.h_kv;
    const int64_t rows = (int64_t)a.B * a.Hq;
    char* ws = static_cast<char*>(a.ws);
    // the split merge: log-sum-exp over splits (a first stage over groups of
    // 32 when there are many), then Pi_v^T and 1/l
    auto merge = [&](MergeK mk, float* part, int nsplit, int width) -> hipError_t {
        mk.part = part;
        mk.nsplit = nsplit;
        if (nsplit > 2 * kMergeGroup) {
            const int ngroup = (nsplit + kMergeGroup - 1) / kMergeGroup;
            float* part2 = part + align256(rows * nsplit * width * 4) / 4;
            const unsigned threads = (unsigned)std::min(512, (width + 63) / 64 * 64);
            hipLaunchKernelGGL(decode_merge_group_kernel, dim3((unsigned)rows, (unsigned)ngroup), dim3(threads), 0, stream,
                               part, nsplit, width, part2, ngroup);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            mk.part = part2;
            mk.nsplit = ngroup;
        }
        using MFn = void (*)(MergeK);
        MFn fn = nullptr;
        const bool d64 = d == 64;
        switch (mk.m) {
            case 0: fn = d64 ? decode_merge_fast_kernel<64, 0> : decode_merge_fast_kernel<128, 0>; break;
            case 32: fn = d64 ? decode_merge_fast_kernel<64, 32> : decode_merge_fast_kernel<128, 32>; break;
            case 64: fn = d64 ? decode_merge_fast_kernel<64, 64> : decode_merge_fast_kernel<128, 64>; break;
            case 128: fn = d64 ? decode_merge_fast_kernel<64, 128> : decode_merge_fast_kernel<128, 128>; break;
            default: fn = d64 ? decode_merge_kernel<64> : decode_merge_kernel<128>; break;
        }
        hipLaunchKernelGGL(fn, dim3((unsigned)rows), dim3(256), 0, stream, mk);
        return hipGetLastError();
    };
    if (ck->spec.block >= 2) {
        // vector codebooks: q' = Pi_k RoPE(q), split kernel, merge (no correction term)
        if (!vq_attn_supported(ck, cv)) return hipErrorInvalidValue;
        int nsplit = 1, split_len = 0;
        vq_attn_plan(a.L_cap, &nsplit, &split_len);
        float* qp = reinterpret_cast<float*>(ws);
        float* part = reinterpret_cast<float*>(ws + align256(rows * d * 4));
        hipError_t e = launch_qprep_rht(ck, a, qp, nullptr, stream);
        if (e != hipSuccess) return e;
        e = launch_vq_attn_split(ck, cv, k, v, a, qp, part, nsplit, split_len, stream);
        if (e != hipSuccess) return e;
        MergeK mk{};
        mk.d = d;
        mk.m = 0;
        mk.sigma = cv->dev.sigma;
        mk.out = a.out;
        return merge(mk, part, nsplit, 2 + d);
    }
    if (ck->dense || cv->dense || cv->spec.bits != bits || cv->spec.m != m) return hipErrorInvalidValue;
    MergeK mk{};
    mk.d = d;
    mk.m = m;
    mk.sigma = cv->dev.sigma;
    mk.sketch = cv->dev.sketch;
    mk.corr = (float)corr_scale(cv);
    mk.s_ident = sign_corr(cv) ? 1 : 0;
    mk.norot = no_rotation(cv) ? 1 : 0;
    mk.out = a.out;
    if (decode_mfma_supported(ck, cv)) {
        int nsplit = 1, split_len = 0;
        decode_mfma_plan(a.B, a.Hq, a.h_kv, a.L_cap, &nsplit, &split_len);
        const QDigits qd = carve_qdigits(ck, ws, rows);
        float* part = reinterpret_cast<float*>(ws + align256(qdigits_workspace_bytes(ck, rows)));
        hipError_t e = launch_qdigits(ck, a, qd, stream);
        if (e != hipSuccess) return e;
        e = launch_decode_mfma(ck, cv, k, v, a, qd, part, nsplit, split_len, stream);
        if (e != hipSuccess) return e;
        return merge(mk, part, nsplit, 2 + d + m);
    }
    float* qp = reinterpret_cast<float*>(ws);
    float* s = qp + rows * d;
    float* part = reinterpret_cast<float*>(ws + align256(rows * (d + m) * 4));
    hipError_t e = launch_qprep_rht(ck, a, qp, s, stream);
    if (e != hipSuccess) return e;
    const int gt = group_tile(G);
    DecFn fn = pick_decode(d, bits, gt);
    if (!fn) return hipErrorInvalidValue;
    DecK p{};
    p.qp = qp;
    p.s = s;
    p.lv_k = ck->dev.levels;
    p.lv_v = cv->dev.levels;
    p.k_norm = k.norm;
    p.k_rnorm = k.rnorm;
    p.k_codes = k.codes;
    p.k_signs = k.signs;
    p.v_norm = v.norm;
    p.v_rnorm = v.rnorm;
    p.v_codes = v.codes;
    p.v_signs = v.signs;
    p.seq_len = a.seq_len;
    p.Hq = a.Hq;
    p.h_kv = a.h_kv;
    p.L_cap = a.L_cap;
    p.m = m;
    p.ngroups = (G + gt - 1) / gt;
    const int64_t bkg = (int64_t)a.B * a.h_kv * p.ngroups;
    p.nsplit = decode_nsplit(bkg, a.L_cap);
    p.chunk = decode_chunk(a.L_cap, p.nsplit);
    p.scale = a.scale;
    p.part = part;
    const int cw = bits * d / 32;
    const size_t lds = (size_t)(2 * gt * d + 32 + 2 * 256 * gt + 4 * gt + 3 * gt) * 4 + (size_t)256 * (cw + m / 32) * 4;
    hipLaunchKernelGGL(fn, dim3((unsigned)bkg, (unsigned)p.nsplit), dim3(256), lds, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    mk.part = part;
    mk.nsplit = p.nsplit;
    if (d == 64) hipLaunchKernelGGL(decode_merge_kernel<64>, dim3((unsigned)rows), dim3(256), 0, stream, mk);
    else hipLaunchKernelGGL(decode_merge_kernel<128>, dim3((unsigned)rows), dim3(256), 0, stream, mk);
    return hipGetLastError();
}

}  // namespace tq
