// FibQuant vector codebooks on the GPU (FibQuant summary, sections 2.1-2.3):
// the same normalise-rotate interface as the scalar codec, but each block of
// two rotated coordinates is replaced by the index of its nearest codeword in
// a shared codebook of N points of the unit disc (rate log2(N)/2 bits per
// coordinate, fractional and below one bit included).
//
// Encoder: a wave holds 128/d vectors, lane p of a vector holding its block
// p (coordinates 2p, 2p+1).  RoPE pairs (i, i + d/2) sit in lanes p and
// p + d/4 and are exchanged by a lane shuffle; the Walsh-Hadamard transform is
// one in-lane butterfly and log2(d/2) lane-shuffle butterflies.  Each lane then
// scans the codebook (in LDS as {c0, c1, |c|^2 / 2}) for the largest
// <y, c> - |c|^2 / 2, which is the nearest codeword, and the indices are
// packed LSB first through a per-wave LDS word buffer.
// Logit scan: one thread per key; the key's indices pick codewords from LDS
// and their dot products with the queries' q' (broadcast from LDS) give
// nu * sum_j <q'_j, c[idx_j]>.
// Decoder: codewords looked up, inverse Walsh-Hadamard transform and signs,
// scaled by nu.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

// the wave's LDS operations so far have completed (and the compiler moves no
// memory access across this point)
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

struct VqEnc {
    const void* x;
    int64_t s_seq, s_tok, s_head;
    int32_t n_seq, n_tok, h_kv, tok_offset, L_cap;
    int64_t n_vec;
    int32_t append;
    const int32_t* pos;
    const float* rope_cos;
    const float* rope_sin;
    int32_t rope_npos;
    const int32_t* pages;
    int32_t page_size, max_pages;
    int64_t n_pages;
    dev::FastDiv div_page, div_h, div_tok;
    const float* sigma;
    const float* code;  // [N][2]
    int32_t N, bits, words;
    float* norm;
    uint32_t* codes;
};

template <int D, bool BF16>
__global__ __launch_bounds__(256) void vq_encode_kernel(VqEnc p) {
    constexpr int LPV = D / 2;    // lanes per vector
    constexpr int VPW = 64 / LPV; // vectors per wave
    __shared__ float4 s_code[256];
    __shared__ uint32_t s_words[4][VPW * 16];
    for (int i = threadIdx.x; i < p.N; i += blockDim.x) {
        const float c0 = p.code[2 * i], c1 = p.code[2 * i + 1];
        s_code[i] = make_float4(c0, c1, 0.5f * (c0 * c0 + c1 * c1), 0.0f);
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pl = lane % LPV;      // block index within the vector
    const int vw = lane / LPV;      // vector within the wave
    const float sg0 = p.sigma[2 * pl], sg1 = p.sigma[2 * pl + 1];
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    uint32_t* words = s_words[wave] + vw * 16;
    const int64_t stride = (int64_t)gridDim.x * 4 * VPW;
    for (int64_t v0 = ((int64_t)blockIdx.x * 4 + wave) * VPW; v0 < p.n_vec; v0 += stride) {
        const int64_t vid = min(v0 + vw, p.n_vec - 1);
        bool valid = v0 + vw < p.n_vec;
        // the vector's input, its cache slot and its RoPE row
        int seq, head;
        int64_t slot, in_off;
        int rpos;
        const uint32_t r = p.div_h.div((uint32_t)vid);
        head = (int)((uint32_t)vid - r * (uint32_t)p.h_kv);
        if (p.append) {
            seq = (int)r;
            slot = p.pos[seq];
            rpos = (int)min(max(slot, (int64_t)0), (int64_t)max(p.rope_npos - 1, 0));
            in_off = (int64_t)seq * p.s_seq + (int64_t)head * p.s_head;
        } else {
            const uint32_t sq = p.div_tok.div(r);
            const int tok = (int)(r - sq * (uint32_t)p.n_tok);
            seq = (int)sq;
            slot = (int64_t)p.tok_offset + tok;
            rpos = (int)slot;
            in_off = (int64_t)seq * p.s_seq + (int64_t)tok * p.s_tok + (int64_t)head * p.s_head;
        }
        int64_t rec = -1;
        if (p.pages) {
            if (slot >= 0 && slot < (int64_t)p.max_pages * p.page_size) {
                const uint32_t j = p.div_page.div((uint32_t)slot);
                const int32_t pg = p.pages[(int64_t)seq * p.max_pages + j];
                if (pg >= 0 && pg < p.n_pages) rec = ((int64_t)pg * p.h_kv + head) * p.page_size + (slot - (int64_t)j * p.page_size);
            }
        } else if (slot >= 0 && slot < p.L_cap) {
            rec = ((int64_t)seq * p.h_kv + head) * p.L_cap + slot;
        }
        valid = valid && rec >= 0;
        float a, b;
        if constexpr (BF16) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.x) + in_off + 2 * pl);
            a = __uint_as_float(w << 16);
            b = __uint_as_float(w & 0xFFFF0000u);
        } else {
            const float2 w = *reinterpret_cast<const float2*>(static_cast<const float*>(p.x) + in_off + 2 * pl);
            a = w.x;
            b = w.y;
        }
        if (p.rope_cos) {
            // pair (i, i + D/2): lanes pl and pl + D/4 of the vector
            const float pa = __shfl_xor(a, D / 4), pb = __shfl_xor(b, D / 4);
            const bool lo = pl < D / 4;
            const int64_t ti = (int64_t)rpos * (D / 2) + 2 * (lo ? pl : pl - D / 4);
            const float c0 = p.rope_cos[ti], c1 = p.rope_cos[ti + 1];
            const float s0 = p.rope_sin[ti], s1 = p.rope_sin[ti + 1];
            if (lo) {
                a = fmaf(a, c0, -(pa * s0));
                b = fmaf(b, c1, -(pb * s1));
            } else {
                a = fmaf(a, c0, pa * s0);
                b = fmaf(b, c1, pb * s1);
            }
        }
        float ss = fmaf(a, a, b * b);
#pragma unroll
        for (int m = 1; m < LPV; m <<= 1) ss += __shfl_xor(ss, m);
        const float nu = sqrtf(ss);
        const float sc = nu > 0.0f ? 1.0f / nu : 0.0f;
        a = a * sc * sg0;
        b = b * sc * sg1;
        // Walsh-Hadamard: coordinate stride 1 in the lane, strides 2m across lanes
        {
            const float t = a + b;
            b = a - b;
            a = t;
        }
#pragma unroll
        for (int m = 1; m < LPV; m <<= 1) {
            const float qa = __shfl_xor(a, m), qb = __shfl_xor(b, m);
            if (pl & m) {
                a = qa - a;
                b = qb - b;
            } else {
                a = a + qa;
                b = b + qb;
            }
        }
        // + 0: a zero vector's -0 coordinates count as +0
        const float y0 = a * inv_sqrt_d + 0.0f, y1 = b * inv_sqrt_d + 0.0f;
        // nearest codeword: the largest <y, c> - |c|^2 / 2 (ties to the smaller index)
        int best = 0;
        float bs = -INFINITY;
        for (int n = 0; n < p.N; ++n) {
            const float4 c = s_code[n];
            const float sn = fmaf(c.x, y0, fmaf(c.y, y1, -c.z));
            if (sn > bs) {
                bs = sn;
                best = n;
            }
        }
        // pack: index pl at bits [pl*bits, (pl+1)*bits) of the vector's words
        if (pl < 16) words[pl] = 0u;
        lds_wait();
        const int o = pl * p.bits, wi = o >> 5, sh = o & 31;
        atomicOr(&words[wi], (uint32_t)best << sh);
        if (sh + p.bits > 32) atomicOr(&words[wi + 1], (uint32_t)best >> (32 - sh));
        lds_wait();
        if (valid) {
            if (pl < p.words) p.codes[rec * p.words + pl] = words[pl];
            if (pl == 0) p.norm[rec] = nu;
        }
        lds_wait();
    }
}

struct VqLog {
    const float* qp;  // [B*Hq][D]
    const float* norm;
    const uint32_t* codes;
    const float* code;  // [N][2]
    const int32_t* seq_len;
    int32_t Hq, h_kv, L_cap, N, words, ngroups;
    int32_t k0, klen;
    float* out;
    int64_t ld;
    int32_t col0;
    const int32_t* pages;
    int32_t page_size, max_pages;
    int64_t n_pages;
    dev::FastDiv div_page;
};

constexpr int kVqGroup = 8;  // queries per block

template <int D, int BITS>
__global__ __launch_bounds__(256) void vq_logits_kernel(VqLog p) {
    constexpr int NB = D / 2;
    constexpr int W = (NB * BITS + 31) / 32;
    __shared__ float2 s_code[256];
    __shared__ float2 s_q[kVqGroup][NB];
    const int grp = blockIdx.x % p.ngroups;
    const int64_t bk = blockIdx.x / p.ngroups;
    const int b = (int)(bk / p.h_kv), kh = (int)(bk % p.h_kv);
    const int G = p.Hq / p.h_kv;
    const int g0 = grp * kVqGroup;
    const int ng = min(kVqGroup, G - g0);
    const int64_t row0 = (int64_t)b * p.Hq + (int64_t)kh * G + g0;
    for (int i = threadIdx.x; i < p.N; i += blockDim.x) s_code[i] = make_float2(p.code[2 * i], p.code[2 * i + 1]);
    for (int i = threadIdx.x; i < kVqGroup * NB; i += blockDim.x) {
        const int g = i / NB, j = i % NB;
        s_q[g][j] = g < ng ? make_float2(p.qp[(row0 + g) * D + 2 * j], p.qp[(row0 + g) * D + 2 * j + 1])
                           : make_float2(0.f, 0.f);
    }
    __syncthreads();
    const int sl = min(max(p.seq_len[b], 0), p.L_cap);
    const int t = p.k0 + blockIdx.y * blockDim.x + threadIdx.x;
    if (t >= min(sl, p.k0 + p.klen)) return;
    int64_t rec;
    if (p.pages) {
        const uint32_t j = p.div_page.div((uint32_t)t);
        int64_t pg = p.pages[(int64_t)b * p.max_pages + j];
        pg = pg < 0 ? 0 : (pg >= p.n_pages ? p.n_pages - 1 : pg);
        rec = (pg * p.h_kv + kh) * p.page_size + (t - (int64_t)j * p.page_size);
    } else {
        rec = bk * p.L_cap + t;
    }
    uint32_t w[W];
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = p.codes[rec * W + i];
    const float nu = p.norm[rec];
    float acc[kVqGroup];
#pragma unroll
    for (int g = 0; g < kVqGroup; ++g) acc[g] = 0.f;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        constexpr uint32_t MASK = (1u << BITS) - 1u;
        const int o = j * BITS;
        uint32_t idx = w[o >> 5] >> (o & 31);
        if ((o & 31) + BITS > 32) idx |= w[(o >> 5) + 1] << (32 - (o & 31));
        const float2 c = s_code[idx & MASK];
#pragma unroll
        for (int g = 0; g < kVqGroup; ++g) acc[g] = fmaf(c.x, s_q[g][j].x, fmaf(c.y, s_q[g][j].y, acc[g]));
    }
#pragma unroll
    for (int g = 0; g < kVqGroup; ++g)
        if (g < ng) p.out[(row0 + g) * p.ld + (t - p.col0)] = acc[g] * nu;
}

struct VqDec {
    const float* norm;
    const uint32_t* codes;
    const float* code;
    const float* sigma;
    int32_t N, bits, words;
    int64_t first, count;
    float* out;  // [count][D]
};

template <int D>
__global__ __launch_bounds__(256) void vq_decode_kernel(VqDec p) {
    constexpr int LPV = D / 2, VPW = 64 / LPV;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pl = lane % LPV, vw = lane / LPV;
    const float sg0 = p.sigma[2 * pl], sg1 = p.sigma[2 * pl + 1];
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    const int64_t stride = (int64_t)gridDim.x * 4 * VPW;
    for (int64_t v0 = ((int64_t)blockIdx.x * 4 + wave) * VPW; v0 < p.count; v0 += stride) {
        const int64_t i = min(v0 + vw, p.count - 1);
        const int64_t rec = p.first + i;
        const int o = pl * p.bits;
        uint32_t idx = p.codes[rec * p.words + (o >> 5)] >> (o & 31);
        if ((o & 31) + p.bits > 32) idx |= p.codes[rec * p.words + (o >> 5) + 1] << (32 - (o & 31));
        idx &= (1u << p.bits) - 1u;
        idx = min(idx, (uint32_t)p.N - 1u);
        float a = p.code[2 * idx], b = p.code[2 * idx + 1];
        {
            const float t = a + b;
            b = a - b;
            a = t;
        }
#pragma unroll
        for (int m = 1; m < LPV; m <<= 1) {
            const float qa = __shfl_xor(a, m), qb = __shfl_xor(b, m);
            if (pl & m) {
                a = qa - a;
                b = qb - b;
            } else {
                a = a + qa;
                b = b + qb;
            }
        }
        const float s = p.norm[rec] * inv_sqrt_d;
        if (v0 + vw < p.count)
            *reinterpret_cast<float2*>(p.out + i * D + 2 * pl) = make_float2(a * sg0 * s, b * sg1 * s);
    }
}

using VqLogFn = void (*)(VqLog);
template <int D>
VqLogFn pick_vq_logits(int bits) {
    switch (bits) {
        case 1: return vq_logits_kernel<D, 1>;
        case 2: return vq_logits_kernel<D, 2>;
        case 3: return vq_logits_kernel<D, 3>;
        case 4: return vq_logits_kernel<D, 4>;
        case 5: return vq_logits_kernel<D, 5>;
        case 6: return vq_logits_kernel<D, 6>;
        case 7: return vq_logits_kernel<D, 7>;
        case 8: return vq_logits_kernel<D, 8>;
    }
    return nullptr;
}

int vq_grid(int64_t waves_needed) {
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 256;
    }
    const int64_t blocks = (waves_needed + 3) / 4;
    return (int)std::max<int64_t>(1, std::min<int64_t>(blocks, (int64_t)cus * 8));
}

}  // namespace

bool vq_supported(const tq_codebook* cb) {
    return cb->spec.block == 2 && !cb->dense && (cb->spec.d == 64 || cb->spec.d == 128);
}

hipError_t launch_vq_encode(const tq_codebook* cb, const EncodeArgs& a, hipStream_t stream) {
    const int d = cb->spec.d;
    VqEnc p{};
    p.x = a.x;
    p.s_seq = a.s_seq;
    p.s_tok = a.s_tok;
    p.s_head = a.s_head;
    p.n_seq = a.n_seq;
    p.n_tok = a.n_tok;
    p.h_kv = a.h_kv;
    p.tok_offset = a.tok_offset;
    p.L_cap = a.L_cap;
    p.n_vec = (int64_t)a.n_seq * a.n_tok * a.h_kv;
    p.append = a.append;
    p.pos = a.pos;
    p.rope_cos = a.rope_cos;
    p.rope_sin = a.rope_sin;
    p.rope_npos = a.rope_npos;
    p.pages = a.pages.table;
    p.page_size = a.pages.size;
    p.max_pages = a.pages.max_pages;
    p.n_pages = a.pages.n_pages;
    p.div_page = dev::FastDiv((uint32_t)(a.pages.size > 0 ? a.pages.size : 1));
    p.div_h = dev::FastDiv((uint32_t)a.h_kv);
    p.div_tok = dev::FastDiv((uint32_t)(a.n_tok > 0 ? a.n_tok : 1));
    p.sigma = cb->dev.sigma;
    p.code = cb->dev.levels;
    p.N = cb->K;
    p.bits = cb->spec.bits;
    p.words = (int)((cb->spec.bits * (d / 2) + 31) / 32);
    p.norm = a.out.norm;
    p.codes = a.out.codes;
    const int vpw = 128 / d;
    const int grid = vq_grid((p.n_vec + vpw - 1) / vpw);
    if (d == 64) {
        if (a.bf16) hipLaunchKernelGGL((vq_encode_kernel<64, true>), dim3(grid), dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((vq_encode_kernel<64, false>), dim3(grid), dim3(256), 0, stream, p);
    } else {
        if (a.bf16) hipLaunchKernelGGL((vq_encode_kernel<128, true>), dim3(grid), dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((vq_encode_kernel<128, false>), dim3(grid), dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_vq_logits(const tq_codebook* ck, const tq_packed& k, const AttnArgs& a, const float* qp, int k0,
                            int klen, float* out, int64_t ld, int col0, hipStream_t stream) {
    const int d = ck->spec.d;
    VqLogFn fn = d == 64 ? pick_vq_logits<64>(ck->spec.bits) : pick_vq_logits<128>(ck->spec.bits);
    if (!fn) return hipErrorInvalidValue;
    const int G = a.Hq / a.h_kv;
    VqLog p{};
    p.qp = qp;
    p.norm = k.norm;
    p.codes = k.codes;
    p.code = ck->dev.levels;
    p.seq_len = a.seq_len;
    p.Hq = a.Hq;
    p.h_kv = a.h_kv;
    p.L_cap = a.L_cap;
    p.N = ck->K;
    p.words = (int)((ck->spec.bits * (d / 2) + 31) / 32);
    p.ngroups = (G + kVqGroup - 1) / kVqGroup;
    p.k0 = k0;
    p.klen = klen;
    p.out = out;
    p.ld = ld;
    p.col0 = col0;
    p.pages = a.pages.table;
    p.page_size = a.pages.size;
    p.max_pages = a.pages.max_pages;
    p.n_pages = a.pages.n_pages;
    p.div_page = dev::FastDiv((uint32_t)(a.pages.size > 0 ? a.pages.size : 1));
    const int64_t gx = (int64_t)a.B * a.h_kv * p.ngroups;
    const int64_t gy = (klen + 255) / 256;
    if (gx == 0 || gy == 0) return hipSuccess;
    hipLaunchKernelGGL(fn, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_vq_decode(const tq_codebook* cb, const tq_packed& k, int64_t first, int64_t count, float* out,
                            hipStream_t stream) {
    const int d = cb->spec.d;
    VqDec p{};
    p.norm = k.norm;
    p.codes = k.codes;
    p.code = cb->dev.levels;
    p.sigma = cb->dev.sigma;
    p.N = cb->K;
    p.bits = cb->spec.bits;
    p.words = (int)((cb->spec.bits * (d / 2) + 31) / 32);
    p.first = first;
    p.count = count;
    p.out = out;
    const int vpw = 128 / d;
    const int grid = vq_grid((count + vpw - 1) / vpw);
    if (count == 0) return hipSuccess;
    if (d == 64) hipLaunchKernelGGL(vq_decode_kernel<64>, dim3(grid), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL(vq_decode_kernel<128>, dim3(grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace tq
