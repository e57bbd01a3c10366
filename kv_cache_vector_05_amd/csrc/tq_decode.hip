// Fused decode on the integer matrix cores: softmax(scale * logits) times
// values, straight from packed keys and values.
//
// TurboESM summary, technical section 2: dequantisation, the residual
// correction and the softmax run in one kernel, with no dequantised copy of
// the cache.  Per query, the split kernel returns for its share of the key
// axis the max logit M, l = sum_j exp(a_j - M) and, in the rotated domain,
//     A_y[i] = sum_j w_j t_v[c_ji],   A_z[r] = sum_j w_j gamma_j z_jr,   w_j = exp(a_j - M) nu_j
// (with the sign correction of the TurboESM summary, technical section 2,
// gamma_j is the KV head's mu and S_v = I);
// the merge kernel combines the splits by log-sum-exp and maps back once per
// query: out = Pi_v^T (A_y + sqrt(pi/2)/m S_v^T A_z) / l  (iaemfoco post,
// "TurboQuant: Uma Nova Abordagem", the QJL dequantiser; FibQuant summary,
// section 2.3: lookup, inverse rotation, norm scale).
//
// A workgroup (four waves) owns one split of at most 512 keys of one KV head
// and makes two passes over it:
//  1. the logit of every key with the exact int8-MFMA tile of the scan (one
//     16-key tile per wave per 64 keys), kept in LDS, plus the split's max
//     logit per query and the max of nu and nu*gamma over its values;
//  2. per 64 keys: the weights w and w*gamma as 28-bit fixed point (one scale
//     per split) in four balanced base-128 digits, the value levels' three
//     base-256 digits and the sign bits as +-1 bytes, each written to LDS as
//     one 16-byte row per key.  ds_read_b64_tr_b8 reads them back transposed
//     (keys along K) as the operands of v_mfma_i32_16x16x64_i8: rows =
//     (query, digit of w), columns = 16 coordinates, K = 64 keys.  Each wave
//     accumulates a quarter of the columns.  The integer sums are exact and
//     carried across the split; only the final digit combination is rounded.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

using dev::intx2;
using dev::intx4;
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct DecM {
    const int8_t* qd;
    const int8_t* sd;
    const float* qscale;
    int32_t sdw;
    const float* k_norm;
    const float* k_rnorm;
    const uint32_t* k_codes;
    const uint32_t* k_signs;
    const float* v_norm;
    const float* v_rnorm;
    const uint32_t* v_codes;
    const uint32_t* v_signs;
    const int32_t* seq_len;
    int32_t Hq, h_kv, L_cap, ngroups, nsplit, split_len;
    float scale;
    uint32_t tdig_k[16];
    int32_t shift_k;
    uint32_t tdig_v[16];
    int32_t shift_v;
    double cq_k;                  // scale of the key correction term
    const float* k_mu;            // sign correction: mu per KV head, else nullptr (gamma per key)
    const float* v_mu;
    int32_t k_mu_stride, v_mu_stride;
    // paged records (pages != nullptr): page table [B][max_pages] of pages of
    // page_size slots, a multiple of 64, so a 64-key chunk (splits start at
    // multiples of 64) lies in one page; entries are clamped into [0, n_pages)
    const int32_t* pages;
    int32_t page_size, max_pages;
    int64_t n_pages;
    dev::FastDiv div_page;
    float* part;  // [B*Hq][nsplit][2 + D + M]
};

// keys per split at most: the logits and weight digits of a split stay in
// LDS (24 KB per row tile of four queries at 512 keys)
template <int NRT>
constexpr int split_max() {
    return NRT == 1 ? 512 : 256;
}

typedef __attribute__((address_space(3))) intx2* lds_intx2_ptr;

// One MFMA operand from a [64 keys][16 bytes] block in LDS: lane l receives
// byte (l % 16) of the rows of keys 8 (l/16) .. +7 and 32 + 8 (l/16) .. +7.
// Both operands of a product are read this way, so their K slots agree.
__device__ __forceinline__ intx4 tr_operand(const int8_t* blk, int lane) {
    const intx2 lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_intx2_ptr)(blk + 8 * lane));
    const intx2 hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_intx2_ptr)(blk + 512 + 8 * lane));
    return intx4{lo[0], lo[1], hi[0], hi[1]};
}

// four base-128 digits (0..127, most significant in byte 0) of 0 <= X < 2^28:
// the weights are non-negative, so no balancing is needed
__device__ __forceinline__ uint32_t digits4_unsigned(uint32_t X) {
    return ((X >> 21) & 0x7Fu) | ((X >> 6) & 0x7F00u) | ((X << 9) & 0x7F0000u) | ((X << 24) & 0x7F000000u);
}

// value of four rows holding the base-128 digits of one operand (double: the
// sums of a whole split can exceed the int32 range once scaled by 128)
__device__ __forceinline__ double digit_rows(const intx4& a) {
    return ((double)a[0] * 2097152.0 + (double)a[1] * 16384.0) + ((double)a[2] * 128.0 + (double)a[3]);
}

__device__ __forceinline__ float max16(float v) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float sum16(float v) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ float max64(float v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float sum64(float v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
    return v;
}

template <int D, int BITS, int NRT, int M, bool PAGED>
// One row tile runs five waves per SIMD: with one operand block per wave's
// buffer (28 KB of LDS) and at most 96 VGPRs, five four-wave workgroups share
// a CU (measured 3 % faster than four).  Two row tiles (33 KB of LDS) run
// four, held to 128 VGPRs (measured 2 % faster than the three their 138
// VGPRs would give).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NRT == 1 ? 5 : 4))) void decode_mfma_kernel(
    DecM p) {
    constexpr int NCS = M == 0 ? 0 : (M >= 64 ? M / 64 : 1);  // K=64 sketch chunks of the logit
    using TL = dev::TileLogit<D, BITS, NRT, NCS>;
    using Q = typename TL::Q;
    constexpr int SMAX = split_max<NRT>();
    constexpr int NCH = SMAX / 64;        // 64-key chunks per split at most
    constexpr int KPT = SMAX / 256;       // keys per thread in the weight pass
    constexpr int CBW = D / 64;           // 16-coordinate column blocks of A_y per coordinate quarter
    constexpr int PER = M / 4;            // sketch rows per coordinate quarter
    constexpr int ZBW = (PER + 15) / 16;  // 16-row column blocks of A_z per quarter
    constexpr int MW = M / 32;            // sign words per record
    constexpr int NWO = M > 0 ? 2 : 1;    // weight operands: w (and w * gamma)
    static_assert(ZBW <= CBW, "the operand buffer holds CBW blocks");
    // operand blocks per wave's B buffer: one row tile passes its blocks
    // through one block in turn (less LDS, a fifth workgroup per CU); two
    // row tiles write all CBW blocks before reading them back
    constexpr int NBB = NRT == 1 ? 1 : CBW;
    // record loads run this many 64-key chunks ahead of their use
    constexpr int KDEPTH = 4, VDEPTH = 4;

    // logits of the split [rt][chunk][key][query of the row tile]
    __shared__ f32x4 lgs[NRT * NCH * 64];
    // weight digits of the split: A-operand rows [w | w gamma][rt][chunk][key][16]
    __shared__ __attribute__((aligned(16))) int8_t wdig[NWO * NRT * NCH * 1024];
    // per wave: one B-operand buffer [block][key][16] that the level digits
    // and the sign bytes pass through in turn
    __shared__ __attribute__((aligned(16))) int8_t bpool[4 * NBB * 1024];
    __shared__ float red[32 * NRT + 8];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int n = lane & 15;
    const int qk = lane >> 4;
    const int grp = blockIdx.x % p.ngroups;
    const int64_t bk = blockIdx.x / p.ngroups;
    const int b = (int)(bk / p.h_kv);
    const int kh = (int)(bk % p.h_kv);
    const int G = p.Hq / p.h_kv;
    const int64_t rowbase = (int64_t)b * p.Hq + (int64_t)kh * G;
    const int gq0 = grp * 4 * NRT;
    const int split = blockIdx.y;
    constexpr int width = 2 + D + M;

    const int sl = dev::clamp_len(p.seq_len, b, p.L_cap);
    const int c0 = split * p.split_len;
    const int c1 = min(c0 + p.split_len, sl);
    if (c0 >= c1) {  // empty split: weight 0 in the merge, all-zero columns
        for (int i = t; i < 4 * NRT * width; i += blockDim.x) {
            const int g = gq0 + i / width, c = i % width;
            if (g < G) p.part[((rowbase + g) * p.nsplit + split) * width + c] = c == 0 ? -INFINITY : 0.f;
        }
        return;
    }
    const int nch = (c1 - c0 + 63) / 64;
    const int64_t rec_base = bk * p.L_cap;
    // record index of key c0 + 64 c + r (0 <= r < 64) of this (sequence, KV head)
    auto record = [&](int c, int r) -> int64_t {
        if constexpr (PAGED) {
            const int key0 = __builtin_amdgcn_readfirstlane(c0 + 64 * c);
            const uint32_t j = p.div_page.div((uint32_t)key0);
            int64_t pg = p.pages[(int64_t)b * p.max_pages + j];
            pg = pg < 0 ? 0 : (pg >= p.n_pages ? p.n_pages - 1 : pg);
            return (pg * p.h_kv + kh) * p.page_size + (key0 - (int64_t)j * p.page_size) + r;
        }
        return rec_base + c0 + 64 * c + r;
    };
    // record of row r of chunk c; chunks past the split's last one, and rows
    // past its last key, reload the last key's record (unused), so the loads
    // need no branch and can all be in flight together
    auto rec_of = [&](int c, int r) -> int64_t {
        const int cc = min(c, nch - 1);
        return record(cc, min(r, c1 - 1 - c0 - 64 * cc));
    };
    // correction weights: gamma per record (QJL sketch) or the KV head's mu.
    // Loads are unconditional (a resource of size zero reads zeros where a
    // plane is absent) and a weight is the sum of the two readings, so no
    // load sits behind a branch and every wait counts exactly.
    const int64_t kmu = (int64_t)kh * p.k_mu_stride, vmu = (int64_t)kh * p.v_mu_stride;
    const float k_head = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(dev::buf_rsrc(p.k_mu ? p.k_mu + kmu : nullptr, p.k_mu ? 4 : 0), 0, 0, 0));
    const float v_head = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(dev::buf_rsrc(p.v_mu ? p.v_mu + vmu : nullptr, p.v_mu ? 4 : 0), 0, 0, 0));
    // contiguous records: one buffer resource per plane over the split's
    // records, so that every load is a fixed lane offset plus a scalar one
    // (keys past the split read zeros, which no output uses)
    const int64_t recs = rec_base + c0;
    const int64_t nkeys = c1 - c0;
    constexpr int CW = Q::CW;
    __amdgpu_buffer_rsrc_t kc = dev::buf_rsrc(nullptr, 0), ks = kc, kn = kc, kg = kc, vc = kc, vs = kc, vn = kc, vg = kc;
    if constexpr (!PAGED) {
        kc = dev::buf_rsrc(p.k_codes + recs * CW, nkeys * CW * 4);
        kn = dev::buf_rsrc(p.k_norm + recs, nkeys * 4);
        vc = dev::buf_rsrc(p.v_codes + recs * CW, nkeys * CW * 4);
        vn = dev::buf_rsrc(p.v_norm + recs, nkeys * 4);
        if constexpr (M > 0) {
            ks = dev::buf_rsrc(p.k_signs + recs * MW, nkeys * MW * 4);
            vs = dev::buf_rsrc(p.v_signs + recs * MW, nkeys * MW * 4);
            if (!p.k_mu) kg = dev::buf_rsrc(p.k_rnorm + recs, nkeys * 4);
            if (!p.v_mu) vg = dev::buf_rsrc(p.v_rnorm + recs, nkeys * 4);
        }
    }

    // the value norms of the keys this thread weighs (key t + 256 i of the split)
    float vnw[KPT], vgw[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int kk = t + 256 * i;
        if constexpr (PAGED) {
            const int64_t rec = rec_of(kk >> 6, kk & 63);
            vnw[i] = p.v_norm[rec];
            vgw[i] = M > 0 ? (p.v_mu ? v_head : p.v_rnorm[rec]) : 0.f;
        } else {
            vnw[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(vn, 4u * kk, 0, 0));
            vgw[i] = M > 0 ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(vg, 4u * kk, 0, 0)) + v_head : 0.f;
        }
    }

    // ---------------- pass 1: logits, split max, value-norm bounds
    // lane (qk, n) of wave w scores key 16 w + n of every chunk for query qk
    // of each row tile; the key records run KDEPTH chunks ahead
    const int row1 = 16 * wave + n;
    float mx[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) mx[rt] = -INFINITY;
    {
        TL tl;
        tl.init(p.qd, p.sd, p.qscale, p.sdw, p.cq_k, rowbase, gq0, G, p.tdig_k, p.shift_k, lane);
        struct Rec1 {
            typename TL::Raw raw;
            float nu, gm;
        } kr[NCH];
        auto fetch1 = [&](int c) {
            if constexpr (PAGED) {
                const int64_t rec = rec_of(c, row1);
                TL::load(p.k_codes + rec * Q::CW + Q::word0(qk), p.k_signs + rec * MW, PER, lane, kr[c].raw);
                kr[c].nu = p.k_norm[rec];
                kr[c].gm = M > 0 ? (p.k_mu ? k_head : p.k_rnorm[rec]) : 0.f;
            } else {
                const uint32_t key = (uint32_t)(64 * c);  // scalar: the chunk's first key
                dev::quarter_load_buf<D, BITS>(kc, (uint32_t)(row1 * CW + Q::word0(qk)) * 4u, key * CW * 4u, qk,
                                               kr[c].raw.W);
                kr[c].raw.sg = M > 0 ? __builtin_amdgcn_raw_buffer_load_b32(ks, (uint32_t)(row1 * MW + ((qk * PER) >> 5)) * 4u,
                                                                             key * MW * 4u, 0)
                                     : 0u;
                kr[c].nu = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(kn, 4u * row1, 4u * key, 0));
                kr[c].gm = M > 0 ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(kg, 4u * row1, 4u * key, 0)) + k_head
                                 : 0.f;
            }
        };
#pragma unroll
        for (int c = 0; c < KDEPTH && c < NCH; ++c) fetch1(c);
        float* lgf = reinterpret_cast<float*>(lgs);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            // every wave scores its keys of every chunk, also past the split's
            // end (zeros, never used): with no branch around the tile, the
            // records' loads are not moved behind one, where the wait for a
            // chunk would also wait for the chunks fetched after it
            const int key0 = c0 + 64 * c + 16 * wave;
            float a[NRT];
            {
                // keys past the end: + -inf (an add, not a select, so that the
                // compiler does not put the norm loads behind a branch either)
                const float off = key0 + n < c1 ? 0.0f : -INFINITY;
                float lg[NRT];
                tl.compute(kr[c].raw, kr[c].gm, PER, lane, lg);
                const float snu = p.scale * kr[c].nu;
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt) a[rt] = snu * lg[rt] + off;
            }
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                lgf[((rt * NCH + c) * 64 + row1) * 4 + qk] = a[rt];
                mx[rt] = fmaxf(mx[rt], a[rt]);
            }
            if (c + KDEPTH < NCH) fetch1(c + KDEPTH);
        }
    }
    float numax = 0.f, ngmax = 0.f;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        if (c0 + t + 256 * i < c1) {
            numax = fmaxf(numax, vnw[i]);
            ngmax = fmaxf(ngmax, vnw[i] * vgw[i]);
        }
    }

    // value records for pass 2: lane l of every wave takes key l of each
    // chunk, wave w the code words of coordinate quarter w and the sign word
    // of its sketch rows
    struct Rec2 {
        uint32_t W[Q::NW];
        uint32_t sg;
    } vr[NCH];
    auto fetch2 = [&](int c) {
        if constexpr (PAGED) {
            const int64_t rec = rec_of(c, lane);
            Q::load(p.v_codes + rec * Q::CW + Q::word0(wave), wave, vr[c].W);
            vr[c].sg = M > 0 ? p.v_signs[rec * MW + ((wave * PER) >> 5)] : 0u;
        } else {
            const uint32_t key = (uint32_t)(64 * c);
            dev::quarter_load_buf<D, BITS>(vc, (uint32_t)(lane * CW + Q::word0(wave)) * 4u, key * CW * 4u, wave, vr[c].W);
            vr[c].sg = M > 0 ? __builtin_amdgcn_raw_buffer_load_b32(vs, (uint32_t)(lane * MW + ((wave * PER) >> 5)) * 4u,
                                                                     key * MW * 4u, 0)
                             : 0u;
        }
    };
#pragma unroll
    for (int c = 0; c < VDEPTH && c < NCH; ++c) fetch2(c);

#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        mx[rt] = max16(mx[rt]);
        if (n == 0) red[(wave * NRT + rt) * 4 + qk] = mx[rt];
    }
    numax = max64(numax);
    ngmax = max64(ngmax);
    if (lane == 0) {
        red[32 * NRT + wave] = numax;
        red[32 * NRT + 4 + wave] = ngmax;
    }
    __syncthreads();
    float mq[NRT][4];  // the split max of every query of the row tiles
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            float v = red[rt * 4 + qq];
#pragma unroll
            for (int w = 1; w < 4; ++w) v = fmaxf(v, red[(w * NRT + rt) * 4 + qq]);
            mq[rt][qq] = v;
        }
    numax = fmaxf(fmaxf(red[32 * NRT], red[32 * NRT + 1]), fmaxf(red[32 * NRT + 2], red[32 * NRT + 3]));
    ngmax = fmaxf(fmaxf(red[32 * NRT + 4], red[32 * NRT + 5]), fmaxf(red[32 * NRT + 6], red[32 * NRT + 7]));
    // weights: w = p nu <= max nu, w gamma <= max nu gamma (p <= 1)
    const int sw = dev::fixed_shift(numax);
    const int sz = dev::fixed_shift(ngmax);
    // 2^sw, 2^sz as floats (w * 2^sw < 2^26 is exact; tiny norms clamp the exponent)
    const float wscale = ldexpf(1.0f, min(sw, 126));
    const float zscale = ldexpf(1.0f, min(sz, 126));

    // ---------------- weights, once per (query, key) of the split
    // thread t weighs keys t + 256 i for the four queries of each row tile:
    // w = exp(a - M) nu (and w gamma) in fixed point, the base-128 digits of
    // query qq in bytes 4 qq .. 4 qq + 3 of the key's row (A-operand rows
    // 4 qq + digit); exp(-inf) = 0 past the end
    {
        float ls[NRT][4];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) ls[rt][qq] = 0.f;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int kk = t + 256 * i;
            const int c = kk >> 6, r = kk & 63;
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                const f32x4 a = lgs[(rt * NCH + c) * 64 + r];
                uint32_t dw[4], dz[4];
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const float pj = __expf(a[qq] - mq[rt][qq]);
                    ls[rt][qq] += pj;
                    const float w = pj * vnw[i];
                    dw[qq] = digits4_unsigned((uint32_t)rintf(w * wscale));
                    dz[qq] = M > 0 ? digits4_unsigned((uint32_t)rintf((w * vgw[i]) * zscale)) : 0u;
                }
                *reinterpret_cast<intx4*>(wdig + ((0 * NRT + rt) * NCH + c) * 1024 + 16 * r) =
                    intx4{(int)dw[0], (int)dw[1], (int)dw[2], (int)dw[3]};
                if constexpr (M > 0)
                    *reinterpret_cast<intx4*>(wdig + ((1 * NRT + rt) * NCH + c) * 1024 + 16 * r) =
                        intx4{(int)dz[0], (int)dz[1], (int)dz[2], (int)dz[3]};
            }
        }
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const float s = sum64(ls[rt][qq]);
                if (lane == 0) red[16 * NRT + (wave * NRT + rt) * 4 + qq] = s;
            }
    }
    __syncthreads();

    // ---------------- pass 2: weighted value sums on the matrix cores
    // Each wave sums its coordinate quarter over every key of the split,
    // passing its B operands through a region of LDS of its own (written and
    // read back transposed by the same wave, whose LDS accesses are served in
    // order): no workgroup barrier.
    int8_t* bbuf = bpool + wave * NBB * 1024;
    intx4 accy[NRT][CBW][3];
    intx4 accz[NRT][ZBW > 0 ? ZBW : 1];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
        for (int j = 0; j < CBW; ++j)
#pragma unroll
            for (int bb = 0; bb < 3; ++bb) accy[rt][j][bb] = intx4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < (ZBW > 0 ? ZBW : 1); ++j) accz[rt][j] = intx4{0, 0, 0, 0};
    }
    uint32_t tdv[16];
#pragma unroll
    for (int i = 0; i < (BITS == 4 ? 16 : 8); ++i) tdv[i] = p.tdig_v[i];

#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        if (c >= nch) break;  // the same for the whole workgroup
        if (c + VDEPTH < NCH) fetch2(c + VDEPTH);
        const Rec2& r = vr[c];
        intx4 aw[NRT], az[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            aw[rt] = tr_operand(wdig + ((0 * NRT + rt) * NCH + c) * 1024, lane);
            if constexpr (M > 0) az[rt] = tr_operand(wdig + ((1 * NRT + rt) * NCH + c) * 1024, lane);
        }
        // level digits of quarter `wave`, one digit plane at a time:
        // coordinates 16 j + 4 sg .. + 3 of the quarter in bytes 4 sg .. of block j
        uint32_t sel[CBW][4];
#pragma unroll
        for (int j = 0; j < CBW; ++j)
#pragma unroll
            for (int sg = 0; sg < 4; ++sg) sel[j][sg] = Q::sel(r.W, 4 * j + sg, wave);
#pragma unroll
        for (int bb = 0; bb < 3; ++bb) {
#pragma unroll
            for (int j = 0; j < CBW; ++j) {
                intx4 v;
#pragma unroll
                for (int sg = 0; sg < 4; ++sg) v[sg] = (int)dev::lut<BITS>(tdv, bb, sel[j][sg]);
                *reinterpret_cast<intx4*>(bbuf + (j % NBB) * 1024 + 16 * lane) = v;
                if constexpr (NBB == 1) {
                    // the wave's LDS accesses are served in order: the block is
                    // read back before the next one overwrites it
                    const intx4 bv = tr_operand(bbuf, lane);
#pragma unroll
                    for (int rt = 0; rt < NRT; ++rt)
                        accy[rt][j][bb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aw[rt], bv, accy[rt][j][bb], 0, 0, 0);
                }
            }
            if constexpr (NBB > 1) {
#pragma unroll
                for (int j = 0; j < CBW; ++j) {
                    const intx4 bv = tr_operand(bbuf + j * 1024, lane);
#pragma unroll
                    for (int rt = 0; rt < NRT; ++rt)
                        accy[rt][j][bb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aw[rt], bv, accy[rt][j][bb], 0, 0, 0);
                }
            }
        }
        // sign bits of sketch rows wave*PER + 16 zb .. as +-1 bytes (rows past
        // PER, when PER < 16, are zero bytes)
        if constexpr (M > 0) {
#pragma unroll
            for (int zb = 0; zb < ZBW; ++zb) {
                const uint32_t x = r.sg >> ((wave * PER + 16 * zb) & 31);
                intx4 v;
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) v[s4] = 4 * s4 < PER - 16 * zb ? (int)dev::spread4_pm(x >> (4 * s4)) : 0;
                *reinterpret_cast<intx4*>(bbuf + (zb % NBB) * 1024 + 16 * lane) = v;
                if constexpr (NBB == 1) {
                    const intx4 bz = tr_operand(bbuf, lane);
#pragma unroll
                    for (int rt = 0; rt < NRT; ++rt)
                        accz[rt][zb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(az[rt], bz, accz[rt][zb], 0, 0, 0);
                }
            }
            if constexpr (NBB > 1) {
#pragma unroll
                for (int zb = 0; zb < ZBW; ++zb) {
                    const intx4 bz = tr_operand(bbuf + zb * 1024, lane);
#pragma unroll
                    for (int rt = 0; rt < NRT; ++rt)
                        accz[rt][zb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(az[rt], bz, accz[rt][zb], 0, 0, 0);
                }
            }
        }
    }

    // ---------------- partial results of the split
    const double yscale = ldexp(1.0, -(sw + p.shift_v));
    const double zs = ldexp(1.0, -sz);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        const int g = gq0 + 4 * rt + qk;  // lane's query in the MFMA result rows 4 qk .. 4 qk + 3
        if (g >= G) continue;
        float* dst = p.part + ((rowbase + g) * p.nsplit + split) * width;
        if (wave == 0 && n == 0) {
            float mxq = mq[rt][0];
#pragma unroll
            for (int qq = 1; qq < 4; ++qq) mxq = qk == qq ? mq[rt][qq] : mxq;
            const float* lr = red + 16 * NRT;
            dst[0] = mxq;
            dst[1] = (lr[rt * 4 + qk] + lr[(NRT + rt) * 4 + qk]) + (lr[(2 * NRT + rt) * 4 + qk] + lr[(3 * NRT + rt) * 4 + qk]);
        }
#pragma unroll
        for (int j = 0; j < CBW; ++j) {
            double V = 0.0;
#pragma unroll
            for (int bb = 0; bb < 3; ++bb) V = V * 256.0 + digit_rows(accy[rt][j][bb]);
            dst[2 + 16 * (wave * CBW + j) + n] = (float)(V * yscale);
        }
        if constexpr (M > 0) {
#pragma unroll
            for (int zb = 0; zb < ZBW; ++zb)
                if (16 * zb + n < PER) dst[2 + D + wave * PER + 16 * zb + n] = (float)(digit_rows(accz[rt][zb]) * zs);
        }
    }
}

using DecMFn = void (*)(DecM);

template <int D, int BITS, int NRT, bool PG>
DecMFn pick_m(int m) {
    if constexpr (D == 64) {
        switch (m) {
            case 0: return decode_mfma_kernel<D, BITS, NRT, 0, PG>;
            case 32: return decode_mfma_kernel<D, BITS, NRT, 32, PG>;
            case 64: return decode_mfma_kernel<D, BITS, NRT, 64, PG>;
        }
    } else {
        switch (m) {
            case 0: return decode_mfma_kernel<D, BITS, NRT, 0, PG>;
            case 64: return decode_mfma_kernel<D, BITS, NRT, 64, PG>;
            case 128: return decode_mfma_kernel<D, BITS, NRT, 128, PG>;
        }
    }
    return nullptr;
}
template <int D, int BITS, bool PG>
DecMFn pick_nrt(int nrt, int m) {
    return nrt == 1 ? pick_m<D, BITS, 1, PG>(m) : pick_m<D, BITS, 2, PG>(m);
}
template <int D, bool PG>
DecMFn pick_bits(int bits, int nrt, int m) {
    switch (bits) {
        case 1: return pick_nrt<D, 1, PG>(nrt, m);
        case 2: return pick_nrt<D, 2, PG>(nrt, m);
        case 3: return pick_nrt<D, 3, PG>(nrt, m);
        case 4: return pick_nrt<D, 4, PG>(nrt, m);
    }
    return nullptr;
}

int decode_nrt(int G) { return G <= 4 ? 1 : 2; }

}  // namespace

bool decode_mfma_supported(const tq_codebook* ck, const tq_codebook* cv) {
    if (ck->dense || cv->dense || !logits_mfma_supported(ck)) return false;
    const tq_spec &a = ck->spec, &v = cv->spec;
    if (v.d != a.d || v.bits != a.bits || v.m != a.m) return false;
    return a.m == 0 || a.m == a.d / 2 || a.m == a.d;
}

void decode_mfma_plan(int64_t B, int Hq, int h_kv, int L_cap, int* nsplit, int* split_len) {
    const int G = h_kv > 0 ? Hq / h_kv : 1;
    const int nrt = decode_nrt(G);
    const int smax = nrt == 1 ? split_max<1>() : split_max<2>();
    const int64_t heads = B * h_kv * ((G + 4 * nrt - 1) / (4 * nrt));
    // shortest split (multiple of 64 keys, at least 256) that keeps about
    // 2048 workgroups in flight
    int len = smax;
    while (len > 256 && heads * ((L_cap + len - 1) / len) < 2048) len /= 2;
    *split_len = len;
    *nsplit = std::max(1, (L_cap + len - 1) / len);
}

hipError_t launch_decode_mfma(const tq_codebook* ck, const tq_codebook* cv, const tq_packed& k, const tq_packed& v,
                              const AttnArgs& a, const QDigits& q, float* part, int nsplit, int split_len,
                              hipStream_t stream) {
    const int G = a.Hq / a.h_kv;
    const int nrt = decode_nrt(G);
    DecMFn fn = nullptr;
    const bool paged = a.pages.table != nullptr;
    if (ck->spec.d == 64)
        fn = paged ? pick_bits<64, true>(ck->spec.bits, nrt, ck->spec.m) : pick_bits<64, false>(ck->spec.bits, nrt, ck->spec.m);
    else if (ck->spec.d == 128)
        fn = paged ? pick_bits<128, true>(ck->spec.bits, nrt, ck->spec.m) : pick_bits<128, false>(ck->spec.bits, nrt, ck->spec.m);
    if (!fn) return hipErrorInvalidValue;
    DecM p{};
    p.qd = q.qd;
    p.sd = q.sd;
    p.qscale = q.scale;
    p.sdw = q.sdw;
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
    p.ngroups = (G + 4 * nrt - 1) / (4 * nrt);
    p.nsplit = nsplit;
    p.split_len = split_len;
    p.scale = a.scale;
    for (int i = 0; i < 16; ++i) {
        p.tdig_k[i] = ck->lvl_digits[i];
        p.tdig_v[i] = cv->lvl_digits[i];
    }
    p.shift_k = ck->lvl_shift;
    p.shift_v = cv->lvl_shift;
    p.cq_k = corr_scale(ck);
    const MuRef mk = mu_ref(ck), mv = mu_ref(cv);
    p.k_mu = mk.ptr;
    p.k_mu_stride = mk.stride;
    p.v_mu = mv.ptr;
    p.v_mu_stride = mv.stride;
    p.pages = a.pages.table;
    p.page_size = a.pages.size;
    p.max_pages = a.pages.max_pages;
    p.n_pages = a.pages.n_pages;
    p.div_page = dev::FastDiv((uint32_t)(a.pages.size > 0 ? a.pages.size : 1));
    p.part = part;
    const unsigned gx = (unsigned)((int64_t)a.B * a.h_kv * p.ngroups);
    if (gx == 0 || nsplit == 0) return hipSuccess;
    hipLaunchKernelGGL(fn, dim3(gx, (unsigned)nsplit), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace tq
