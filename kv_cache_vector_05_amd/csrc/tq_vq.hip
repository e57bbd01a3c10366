// FibQuant vector codebooks on the GPU (FibQuant summary, sections 2.1-2.3):
// the same normalise-rotate interface as the scalar codec, but each block of
// two rotated coordinates is replaced by the index of its nearest codeword in
// a shared codebook of N points of the unit disc (rate log2(N)/2 bits per
// coordinate, fractional and below one bit included).
//
// The encoder is the Hadamard encoder's vector-codebook mode (tq_encode.hip):
// the rotation leaves whole two-coordinate blocks in each lane.
//
// Logit scan: the product-code form of the dot product.  A block serves one
// (sequence, KV head), up to 4 or 8 of its query heads and 1024 keys; it first
// tabulates T[j][n] = <q'_j, c_n> for every block j and codeword n (one float4
// per entry: four queries), then each thread scores its keys as
// nu * sum_j T[j][idx_j] - one LDS read and one add per query per block.  All
// addresses of one read lie within the N entries of block j, so a read is
// free of bank conflicts.  Codebooks whose table does not fit in LDS use the
// gather form: codewords looked up and multiplied by q' per key.
// Decoder: codewords looked up, inverse Walsh-Hadamard transform and signs,
// scaled by nu (dense rotations: the product with Pi^T per vector).  With a
// dense rotation the encoder and the scan take the dense GEMM path (the
// encoder's dense_vq_kernel, the scan's codeword dequantisation), for blocks
// of 2 or 3 coordinates.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

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

constexpr int kVqGroup = 8;  // queries per block of the gather form
constexpr int kLutBatch = 4;  // keys per thread whose records are loaded together
constexpr int kLutKeys = 8;   // keys per thread of the table form

// the W code words of a record, with the widest loads its alignment allows
template <int W>
__device__ __forceinline__ void load_words(const uint32_t* src, uint32_t (&w)[W]) {
    if constexpr (W % 4 == 0) {
#pragma unroll
        for (int i = 0; i < W / 4; ++i) {
            const uint4 u = reinterpret_cast<const uint4*>(src)[i];
            w[4 * i] = u.x;
            w[4 * i + 1] = u.y;
            w[4 * i + 2] = u.z;
            w[4 * i + 3] = u.w;
        }
    } else if constexpr (W % 2 == 0) {
#pragma unroll
        for (int i = 0; i < W / 2; ++i) {
            const uint2 u = reinterpret_cast<const uint2*>(src)[i];
            w[2 * i] = u.x;
            w[2 * i + 1] = u.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < W; ++i) w[i] = src[i];
    }
}

// index j of a record (BITS bits at bit j * BITS, LSB first)
template <int BITS, int W>
__device__ __forceinline__ uint32_t index_at(const uint32_t (&w)[W], int j) {
    const int o = j * BITS;
    uint32_t idx = w[o >> 5] >> (o & 31);
    if ((o & 31) + BITS > 32) idx |= w[(o >> 5) + 1] << (32 - (o & 31));
    return idx & ((1u << BITS) - 1u);
}

// record of key t of (sequence b, KV head kh) (paged: page-table entries
// clamped into the pool); P carries the page table and the cache shape
template <class P>
__device__ __forceinline__ int64_t vq_record(const P& p, int64_t bk, int b, int kh, int t) {
    if (p.pages) {
        const uint32_t j = p.div_page.div((uint32_t)t);
        int64_t pg = p.pages[(int64_t)b * p.max_pages + j];
        pg = pg < 0 ? 0 : (pg >= p.n_pages ? p.n_pages - 1 : pg);
        return (pg * p.h_kv + kh) * p.page_size + (t - (int64_t)j * p.page_size);
    }
    return bk * p.L_cap + t;
}

// table form: SLOTS float4 entries per (block, codeword), 4 SLOTS queries
template <int D, int BITS, int SLOTS>
__global__ __launch_bounds__(256) void vq_lut_logits_kernel(VqLog p) {
    constexpr int NB = D / 2, N = 1 << BITS, QB = 4 * SLOTS;
    constexpr int W = (NB * BITS + 31) / 32;
    __shared__ float4 s_lut[SLOTS][NB][N];
    __shared__ float s_q[QB][D];
    const int grp = blockIdx.x % p.ngroups;
    const int64_t bk = blockIdx.x / p.ngroups;
    const int b = (int)(bk / p.h_kv), kh = (int)(bk % p.h_kv);
    const int G = p.Hq / p.h_kv;
    const int g0 = grp * QB;
    const int ng = min(QB, G - g0);
    const int64_t row0 = (int64_t)b * p.Hq + (int64_t)kh * G + g0;
    for (int i = threadIdx.x; i < QB * D; i += blockDim.x) {
        const int g = i / D;
        s_q[g][i % D] = g < ng ? p.qp[(row0 + g) * D + i % D] : 0.0f;
    }
    __syncthreads();
    // entry (slot, j, n): thread e serves codeword n = e % N for every (slot, j)
    // it meets (N divides the 256 threads)
    {
        const int n = threadIdx.x % N;
        const float c0 = p.code[2 * n], c1 = p.code[2 * n + 1];
        for (int e = threadIdx.x; e < SLOTS * NB * N; e += blockDim.x) {
            const int sl = e / (NB * N), j = (e / N) % NB;
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = fmaf(s_q[4 * sl + i][2 * j + 1], c1, s_q[4 * sl + i][2 * j] * c0);
            s_lut[sl][j][n] = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
    __syncthreads();
    const int sl_end = min(max(p.seq_len[b], 0), p.L_cap);
    const int t_end = min(sl_end, p.k0 + p.klen);
    const int tb = p.k0 + blockIdx.y * (256 * kLutKeys) + threadIdx.x;
    for (int k0 = 0; k0 < kLutKeys; k0 += kLutBatch) {
        if (tb + 256 * k0 >= t_end) break;
        // the batch's records in flight together (keys past the end re-read
        // the last key and are not stored)
        uint32_t w[kLutBatch][W];
        float nu[kLutBatch];
#pragma unroll
        for (int kk = 0; kk < kLutBatch; ++kk) {
            const int64_t rec = vq_record(p, bk, b, kh, min(tb + 256 * (k0 + kk), t_end - 1));
            load_words<W>(p.codes + rec * W, w[kk]);
            nu[kk] = p.norm[rec];
        }
#pragma unroll
        for (int kk = 0; kk < kLutBatch; ++kk) {
            const int t = tb + 256 * (k0 + kk);
            float acc[QB];
#pragma unroll
            for (int g = 0; g < QB; ++g) acc[g] = 0.0f;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const uint32_t idx = index_at<BITS, W>(w[kk], j);
#pragma unroll
                for (int sl = 0; sl < SLOTS; ++sl) {
                    const float4 f = s_lut[sl][j][idx];
                    acc[4 * sl] += f.x;
                    acc[4 * sl + 1] += f.y;
                    acc[4 * sl + 2] += f.z;
                    acc[4 * sl + 3] += f.w;
                }
                // the sums are formed here (not sunk into the guarded stores
                // below), so only a word's lookups are in flight at a time
                if ((j & 7) == 7) {
#pragma unroll
                    for (int g = 0; g < QB; ++g) asm volatile("" : "+v"(acc[g]));
                }
            }
            if (t < t_end) {
#pragma unroll
                for (int g = 0; g < QB; ++g)
                    if (g < ng) p.out[(row0 + g) * p.ld + (t - p.col0)] = acc[g] * nu[kk];
            }
        }
    }
}

// gather form: codewords looked up per key and multiplied by q' (LDS broadcast)
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
    const int64_t rec = vq_record(p, bk, b, kh, t);
    uint32_t w[W];
    load_words<W>(p.codes + rec * W, w);
    const float nu = p.norm[rec];
    float acc[kVqGroup];
#pragma unroll
    for (int g = 0; g < kVqGroup; ++g) acc[g] = 0.f;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const float2 c = s_code[index_at<BITS, W>(w, j)];
#pragma unroll
        for (int g = 0; g < kVqGroup; ++g) acc[g] = fmaf(c.x, s_q[g][j].x, fmaf(c.y, s_q[g][j].y, acc[g]));
        // the sums are formed here (not sunk into the guarded stores below)
#pragma unroll
        for (int g = 0; g < kVqGroup; ++g) asm volatile("" : "+v"(acc[g]));
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

// ---------------------------------------------------------------- fused decode
// softmax(scale * logits) . V over one split of keys, for vector-coded keys
// and values (FibQuant summary, sections 2.3 and 5: decompression fused into
// attention).  Grid (B * h_kv * ngroups, nsplit); a block of 256 threads
// serves QB = 4 SLOTS query heads of one KV head and up to kVqSplit keys.
// Pass 1 (one key per thread) scores the keys with the product-code table of
// the scan, keeps the logits in LDS as [key][query] and stages the keys'
// value records and norms in LDS.  Per query the split's max M and
// l = sum exp(a - M) follow, and the weights w = exp(a - M) nu_v.  Pass 2: lane
// j of a key stream owns value block j and accumulates sum_t w_t c_v[idx_j(t)]
// for every query from the staged records; stream s takes keys s, s + KS, ...
// (KS = 256 / (D/2)), and the streams' sums are added through LDS.  The
// partials (M, l, A_y) per (query row, split) go to the split merge, which
// applies Pi_v^T and divides by l.
constexpr int kVqSplit = 256;

struct VqAttn {
    const float* qp;  // [B*Hq][D] q' = Pi_k RoPE(q)
    const float* knorm;
    const uint32_t* kcodes;
    const float* kcode;  // key codewords [NK][2]
    const float* vnorm;
    const uint32_t* vcodes;
    const float* vcode;  // value codewords [NV][2]
    const int32_t* seq_len;
    int32_t Hq, h_kv, L_cap, ngroups, nsplit, split_len;
    int32_t vbits, vwords, nv;
    float scale;
    const int32_t* pages;
    int32_t page_size, max_pages;
    int64_t n_pages;
    dev::FastDiv div_page;
    float* part;  // [B*Hq][nsplit][2 + D]
};

template <int D, int KB, int SLOTS>
__global__ __launch_bounds__(256) void vq_attn_split_kernel(VqAttn p) {
    constexpr int NB = D / 2, NK = 1 << KB, QB = 4 * SLOTS;
    constexpr int KW = (NB * KB + 31) / 32;
    constexpr int KS = 256 / NB;  // key streams of pass 2
    constexpr int LUT_F = 4 * SLOTS * NB * NK;
    constexpr int ACC_F = KS * QB * D;
    constexpr int UNION_F = LUT_F > ACC_F ? LUT_F : ACC_F;
    // the key table (pass 1), later the streams' sums (pass 2)
    __shared__ float4 s_u4[UNION_F / 4];
    __shared__ float s_q[QB][D];
    __shared__ float4 s_w4[kVqSplit][SLOTS];  // [key][query]: logits, then weights
    __shared__ float2 s_vc[256];
    // value records of the split, vwords each (+1: a funnel shift reads one word past the last block)
    __shared__ uint32_t s_vrec[kVqSplit * (D / 2 * 8 / 32) + 1];
    __shared__ float s_vn[kVqSplit];
    __shared__ float s_m[QB], s_l[QB];
    float4* s_lut = s_u4;  // [SLOTS][NB][NK]
    float* s_acc = reinterpret_cast<float*>(s_u4);  // [KS][QB][D]
    float* s_w = reinterpret_cast<float*>(s_w4);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = blockIdx.x % p.ngroups;
    const int64_t bk = blockIdx.x / p.ngroups;
    const int b = (int)(bk / p.h_kv), kh = (int)(bk % p.h_kv);
    const int G = p.Hq / p.h_kv;
    const int g0 = grp * QB;
    const int ng = min(QB, G - g0);
    const int64_t row0 = (int64_t)b * p.Hq + (int64_t)kh * G + g0;
    const int sl = min(max(p.seq_len[b], 0), p.L_cap);
    const int t0 = blockIdx.y * p.split_len;
    const int cnt = max(0, min(p.split_len, sl - t0));  // keys of this split below seq_len

    for (int i = threadIdx.x; i < QB * D; i += blockDim.x) {
        const int g = i / D;
        s_q[g][i % D] = g < ng ? p.qp[(row0 + g) * D + i % D] : 0.0f;
    }
    for (int i = threadIdx.x; i < p.nv; i += blockDim.x) s_vc[i] = make_float2(p.vcode[2 * i], p.vcode[2 * i + 1]);
    __syncthreads();
    {
        const int n = threadIdx.x % NK;
        const float c0 = p.kcode[2 * n], c1 = p.kcode[2 * n + 1];
        for (int e = threadIdx.x; e < SLOTS * NB * NK; e += blockDim.x) {
            const int sl4 = e / (NB * NK), j = (e / NK) % NB;
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = fmaf(s_q[4 * sl4 + i][2 * j + 1], c1, s_q[4 * sl4 + i][2 * j] * c0);
            s_lut[(sl4 * NB + j) * NK + n] = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
    __syncthreads();

    // pass 1: scaled logits (keys past seq_len: -inf)
    for (int i = threadIdx.x; i < p.split_len; i += blockDim.x) {
        float acc[QB];
#pragma unroll
        for (int g = 0; g < QB; ++g) acc[g] = 0.0f;
        if (i < cnt) {
            const int64_t rec = vq_record(p, bk, b, kh, t0 + i);
            uint32_t w[KW];
            load_words<KW>(p.kcodes + rec * KW, w);
            const float f = p.knorm[rec] * p.scale;
            for (int u = 0; u < p.vwords; ++u) s_vrec[i * p.vwords + u] = p.vcodes[rec * p.vwords + u];
            s_vn[i] = p.vnorm[rec];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const uint32_t idx = index_at<KB, KW>(w, j);
#pragma unroll
                for (int sl4 = 0; sl4 < SLOTS; ++sl4) {
                    const float4 t = s_lut[(sl4 * NB + j) * NK + idx];
                    acc[4 * sl4] += t.x;
                    acc[4 * sl4 + 1] += t.y;
                    acc[4 * sl4 + 2] += t.z;
                    acc[4 * sl4 + 3] += t.w;
                }
                if ((j & 7) == 7) {
#pragma unroll
                    for (int g = 0; g < QB; ++g) asm volatile("" : "+v"(acc[g]));
                }
            }
#pragma unroll
            for (int g = 0; g < QB; ++g) acc[g] *= f;
        } else {
#pragma unroll
            for (int g = 0; g < QB; ++g) acc[g] = -INFINITY;
        }
#pragma unroll
        for (int sl4 = 0; sl4 < SLOTS; ++sl4)
            s_w4[i][sl4] = make_float4(acc[4 * sl4], acc[4 * sl4 + 1], acc[4 * sl4 + 2], acc[4 * sl4 + 3]);
    }
    __syncthreads();
    // softmax statistics per query (a split with no keys: M = -inf, l = 0)
    for (int g = wave; g < QB; g += 4) {
        float mx = -INFINITY;
        for (int i = lane; i < cnt; i += 64) mx = fmaxf(mx, s_w[i * QB + g]);
        for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        float l = 0.0f;
        for (int i = lane; i < cnt; i += 64) {
            const float e = expf(s_w[i * QB + g] - mx);
            s_w[i * QB + g] = e;
            l += e;
        }
        for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
        if (lane == 0) {
            s_m[g] = mx;
            s_l[g] = l;
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < cnt; i += blockDim.x) {
        const float nv = s_vn[i];
#pragma unroll
        for (int sl4 = 0; sl4 < SLOTS; ++sl4) {
            float4 w = s_w4[i][sl4];
            w.x *= nv;
            w.y *= nv;
            w.z *= nv;
            w.w *= nv;
            s_w4[i][sl4] = w;
        }
    }
    __syncthreads();

    // pass 2: lane j of stream st accumulates value block j
    const int j = threadIdx.x % NB, st = threadIdx.x / NB;
    const int o = j * p.vbits, wi = o >> 5, sh = o & 31;
    const uint32_t vmask = (1u << p.vbits) - 1u;
    float a0[QB], a1[QB];
#pragma unroll
    for (int g = 0; g < QB; ++g) a0[g] = a1[g] = 0.0f;
#pragma unroll 8
    for (int i = st; i < cnt; i += KS) {
        // the index's bits from the word pair (a funnel shift: no branch for
        // indices that straddle two words)
        const uint32_t* vw = s_vrec + i * p.vwords + wi;
        const uint32_t idx = __builtin_amdgcn_alignbit(vw[1], vw[0], sh) & vmask;
        const float2 c = s_vc[idx];
#pragma unroll
        for (int sl4 = 0; sl4 < SLOTS; ++sl4) {
            const float4 w = s_w4[i][sl4];
            a0[4 * sl4] = fmaf(w.x, c.x, a0[4 * sl4]);
            a1[4 * sl4] = fmaf(w.x, c.y, a1[4 * sl4]);
            a0[4 * sl4 + 1] = fmaf(w.y, c.x, a0[4 * sl4 + 1]);
            a1[4 * sl4 + 1] = fmaf(w.y, c.y, a1[4 * sl4 + 1]);
            a0[4 * sl4 + 2] = fmaf(w.z, c.x, a0[4 * sl4 + 2]);
            a1[4 * sl4 + 2] = fmaf(w.z, c.y, a1[4 * sl4 + 2]);
            a0[4 * sl4 + 3] = fmaf(w.w, c.x, a0[4 * sl4 + 3]);
            a1[4 * sl4 + 3] = fmaf(w.w, c.y, a1[4 * sl4 + 3]);
        }
    }
    // (the table is no longer read: every thread passed the barriers above)
#pragma unroll
    for (int g = 0; g < QB; ++g) {
        s_acc[(st * QB + g) * D + 2 * j] = a0[g];
        s_acc[(st * QB + g) * D + 2 * j + 1] = a1[g];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < QB * D; e += blockDim.x) {
        const int g = e / D, c = e % D;
        if (g >= ng) continue;
        float sum = 0.0f;
#pragma unroll
        for (int q = 0; q < KS; ++q) sum += s_acc[(q * QB + g) * D + c];
        p.part[((row0 + g) * p.nsplit + blockIdx.y) * (2 + D) + 2 + c] = sum;
    }
    if (threadIdx.x < ng) {
        float* dst = p.part + ((row0 + threadIdx.x) * p.nsplit + blockIdx.y) * (2 + D);
        dst[0] = s_m[threadIdx.x];
        dst[1] = s_l[threadIdx.x];
    }
}

using VqAttnFn = void (*)(VqAttn);

// LDS of the decode's key table: at most 32 KiB
constexpr bool attn_lut_fits(int d, int bits, int slots) { return (int64_t)slots * (d / 2) * (1 << bits) * 16 <= 32 * 1024; }

template <int D, int KB>
VqAttnFn pick_vq_attn_bits(int slots) {
    if constexpr (attn_lut_fits(D, KB, 2)) {
        if (slots == 2) return vq_attn_split_kernel<D, KB, 2>;
    }
    if constexpr (attn_lut_fits(D, KB, 1)) {
        if (slots == 1) return vq_attn_split_kernel<D, KB, 1>;
    }
    return nullptr;
}

template <int D>
VqAttnFn pick_vq_attn(int kbits, int slots) {
    switch (kbits) {
        case 1: return pick_vq_attn_bits<D, 1>(slots);
        case 2: return pick_vq_attn_bits<D, 2>(slots);
        case 3: return pick_vq_attn_bits<D, 3>(slots);
        case 4: return pick_vq_attn_bits<D, 4>(slots);
        case 5: return pick_vq_attn_bits<D, 5>(slots);
        case 6: return pick_vq_attn_bits<D, 6>(slots);
    }
    return nullptr;
}

int vq_attn_slots(int d, int kbits, int G) {
    if (G > 4 && attn_lut_fits(d, kbits, 2)) return 2;
    return attn_lut_fits(d, kbits, 1) ? 1 : 0;
}

// dense rotation: x = nu Pi^T y_hat, one block per vector (grid-stride); the
// concatenated codewords y_hat are staged in LDS, and thread c forms output
// coordinate c from column c of Pi (rows read in order, coalesced)
struct VqDenseDec {
    const float* norm;
    const uint32_t* codes;
    const float* code;
    const float* rot;  // Pi [d][d] row-major
    int32_t d, block, bits, words;
    int64_t first, count;
    float* out;  // [count][d]
};

__global__ __launch_bounds__(256) void vq_dense_decode_kernel(VqDenseDec p) {
    __shared__ float s_y[4096];
    const int k = p.block, nb = p.d / k;
    const uint32_t mask = (1u << p.bits) - 1u;
    for (int64_t i = blockIdx.x; i < p.count; i += gridDim.x) {
        const int64_t rec = p.first + i;
        const uint32_t* c = p.codes + rec * p.words;
        __syncthreads();  // the previous vector's reads of s_y are done
        for (int j = threadIdx.x; j < nb; j += blockDim.x) {
            const int o = j * p.bits;
            uint32_t idx = c[o >> 5] >> (o & 31);
            if ((o & 31) + p.bits > 32) idx |= c[(o >> 5) + 1] << (32 - (o & 31));
            idx &= mask;
            for (int t = 0; t < k; ++t) s_y[j * k + t] = p.code[idx * k + t];
        }
        __syncthreads();
        const float nu = p.norm[rec];
        for (int col = threadIdx.x; col < p.d; col += blockDim.x) {
            float acc = 0.0f;
            for (int r = 0; r < p.d; ++r) acc = fmaf(p.rot[(int64_t)r * p.d + col], s_y[r], acc);
            p.out[i * p.d + col] = acc * nu;
        }
    }
}

using VqLogFn = void (*)(VqLog);

// LDS of the table form: SLOTS * D/2 * N float4 entries (at most 48 KiB)
constexpr bool lut_fits(int d, int bits, int slots) { return (int64_t)slots * (d / 2) * (1 << bits) * 16 <= 48 * 1024; }

template <int D, int BITS>
VqLogFn pick_vq_bits(int slots) {
    if constexpr (lut_fits(D, BITS, 2)) {
        if (slots == 2) return vq_lut_logits_kernel<D, BITS, 2>;
    }
    if constexpr (lut_fits(D, BITS, 1)) {
        if (slots == 1) return vq_lut_logits_kernel<D, BITS, 1>;
    }
    if (slots == 0) return vq_logits_kernel<D, BITS>;
    return nullptr;
}

// slots: 1 or 2 for the table form, 0 for the gather form
template <int D>
VqLogFn pick_vq_logits(int bits, int slots) {
    switch (bits) {
        case 1: return pick_vq_bits<D, 1>(slots);
        case 2: return pick_vq_bits<D, 2>(slots);
        case 3: return pick_vq_bits<D, 3>(slots);
        case 4: return pick_vq_bits<D, 4>(slots);
        case 5: return pick_vq_bits<D, 5>(slots);
        case 6: return pick_vq_bits<D, 6>(slots);
        case 7: return pick_vq_bits<D, 7>(slots);
        case 8: return pick_vq_bits<D, 8>(slots);
    }
    return nullptr;
}

// blocks of 256 threads for a grid-stride launch needing `waves_needed` waves
int vq_blocks(int64_t waves_needed) {
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
    if (cb->spec.block < 2) return false;
    // dense rotations (d a multiple of 64, any block) run on the dense GEMM path
    if (cb->dense) return cb->spec.d <= 4096;
    return cb->spec.block == 2 && (cb->spec.d == 64 || cb->spec.d == 128);
}

hipError_t launch_vq_logits(const tq_codebook* ck, const tq_packed& k, const AttnArgs& a, const float* qp, int k0,
                            int klen, float* out, int64_t ld, int col0, hipStream_t stream) {
    const int d = ck->spec.d, bits = ck->spec.bits;
    const int G = a.Hq / a.h_kv;
    // table form when the table fits: 8 queries per block for groups above 4
    int slots = 0;
    if (lut_fits(d, bits, 2) && G > 4) slots = 2;
    else if (lut_fits(d, bits, 1)) slots = 1;
    VqLogFn fn = d == 64 ? pick_vq_logits<64>(bits, slots) : pick_vq_logits<128>(bits, slots);
    if (!fn) return hipErrorInvalidValue;
    const int qb = slots ? 4 * slots : kVqGroup;
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
    p.words = (int)((bits * (d / 2) + 31) / 32);
    p.ngroups = (G + qb - 1) / qb;
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
    const int per_block = slots ? 256 * kLutKeys : 256;
    const int64_t gy = (klen + per_block - 1) / per_block;
    if (gx == 0 || gy == 0) return hipSuccess;
    hipLaunchKernelGGL(fn, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, stream, p);
    return hipGetLastError();
}

bool vq_attn_supported(const tq_codebook* ck, const tq_codebook* cv) {
    if (!vq_supported(ck) || !vq_supported(cv) || ck->dense || cv->dense) return false;
    if (ck->spec.d != cv->spec.d) return false;
    return vq_attn_slots(ck->spec.d, ck->spec.bits, 1) > 0;
}

void vq_attn_plan(int L_cap, int* nsplit, int* split_len) {
    *split_len = kVqSplit;
    *nsplit = std::max(1, (L_cap + kVqSplit - 1) / kVqSplit);
}

hipError_t launch_vq_attn_split(const tq_codebook* ck, const tq_codebook* cv, const tq_packed& k, const tq_packed& v,
                                const AttnArgs& a, const float* qp, float* part, int nsplit, int split_len,
                                hipStream_t stream) {
    const int d = ck->spec.d;
    const int G = a.Hq / a.h_kv;
    const int slots = vq_attn_slots(d, ck->spec.bits, G);
    VqAttnFn fn = d == 64 ? pick_vq_attn<64>(ck->spec.bits, slots) : pick_vq_attn<128>(ck->spec.bits, slots);
    if (!fn) return hipErrorInvalidValue;
    VqAttn p{};
    p.qp = qp;
    p.knorm = k.norm;
    p.kcodes = k.codes;
    p.kcode = ck->dev.levels;
    p.vnorm = v.norm;
    p.vcodes = v.codes;
    p.vcode = cv->dev.levels;
    p.seq_len = a.seq_len;
    p.Hq = a.Hq;
    p.h_kv = a.h_kv;
    p.L_cap = a.L_cap;
    p.ngroups = (G + 4 * slots - 1) / (4 * slots);
    p.nsplit = nsplit;
    p.split_len = split_len;
    p.vbits = cv->spec.bits;
    p.vwords = (int)((cv->spec.bits * (d / 2) + 31) / 32);
    p.nv = cv->K;
    p.scale = a.scale;
    p.pages = a.pages.table;
    p.page_size = a.pages.size;
    p.max_pages = a.pages.max_pages;
    p.n_pages = a.pages.n_pages;
    p.div_page = dev::FastDiv((uint32_t)(a.pages.size > 0 ? a.pages.size : 1));
    p.part = part;
    const int64_t gx = (int64_t)a.B * a.h_kv * p.ngroups;
    if (gx == 0) return hipSuccess;
    hipLaunchKernelGGL(fn, dim3((unsigned)gx, (unsigned)nsplit), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_vq_decode(const tq_codebook* cb, const tq_packed& k, int64_t first, int64_t count, float* out,
                            hipStream_t stream) {
    const int d = cb->spec.d;
    if (count == 0) return hipSuccess;
    if (cb->dense) {
        VqDenseDec p{};
        p.norm = k.norm;
        p.codes = k.codes;
        p.code = cb->dev.levels;
        p.rot = cb->dev.rot;
        p.d = d;
        p.block = cb->spec.block;
        p.bits = cb->spec.bits;
        p.words = (int)((cb->spec.bits * (d / cb->spec.block) + 31) / 32);
        p.first = first;
        p.count = count;
        p.out = out;
        const int grid = (int)std::min<int64_t>(count, 2048);
        hipLaunchKernelGGL(vq_dense_decode_kernel, dim3(grid), dim3(256), 0, stream, p);
        return hipGetLastError();
    }
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
    const int grid = vq_blocks((count + vpw - 1) / vpw);
    if (count == 0) return hipSuccess;
    if (d == 64) hipLaunchKernelGGL(vq_decode_kernel<64>, dim3(grid), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL(vq_decode_kernel<128>, dim3(grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace tq
