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
    uint32_t tdig_k[8];
    int32_t shift_k;
    uint32_t tdig_v[8];
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

template <int NRT>
constexpr int split_max() {
    return 512;
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

template <int D, int BITS, int NRT, int M, bool PAGED>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecM p) {
    constexpr int NCS = M == 0 ? 0 : (M >= 64 ? M / 64 : 1);  // K=64 sketch chunks of the logit
    using TL = dev::TileLogit<D, BITS, NRT, NCS>;
    using Q = typename TL::Q;
    constexpr int SMAX = split_max<NRT>();
    constexpr int NCH = SMAX / 64;     // 64-key chunks per split at most
    constexpr int NCB = D / 16;        // 16-coordinate column blocks of A_y
    constexpr int CBW = NCB / 4;       // ... per wave (= per coordinate quarter)
    constexpr int NZB = M / 16;        // 16-row column blocks of A_z
    constexpr int ZBW = (NZB + 3) / 4; // ... per wave at most
    constexpr int PER = M / 4;         // sketch rows per coordinate quarter
    constexpr int MW = M / 32;         // sign words per record

    __shared__ float lgs[4 * NCH * NRT * 64];                    // pass-1 logits (scaled)
    __shared__ __attribute__((aligned(16))) int8_t vy[3 * NCB * 64 * 16];  // [digit][cb][key][16]
    __shared__ __attribute__((aligned(16))) int8_t vz[(NZB > 0 ? NZB : 1) * 64 * 16];  // [cs][key][16]
    __shared__ __attribute__((aligned(16))) int8_t wd[2 * NRT * 64 * 16];  // [w | w*gamma][rt][key][16]
    __shared__ float red[16 * NRT + 8];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
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
        for (int i = threadIdx.x; i < 4 * NRT * width; i += blockDim.x) {
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
    // correction weights: gamma per record (QJL sketch) or the KV head's mu
    const float k_head = p.k_mu ? p.k_mu[kh * p.k_mu_stride] : 0.f;
    const float v_head = p.v_mu ? p.v_mu[kh * p.v_mu_stride] : 0.f;

    // ---------------- pass 1: logits, split max, value-norm bounds
    float mx[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) mx[rt] = -INFINITY;
    float numax = 0.f, ngmax = 0.f;
    {
        TL tl;
        tl.init(p.qd, p.sd, p.qscale, p.sdw, p.cq_k, rowbase, gq0, G, p.tdig_k, p.shift_k, lane);
        // the key record (and the value norms) of the next chunk's tile are
        // loaded before the current tile computes
        struct Rec1 {
            typename TL::Raw raw;
            float nu, gm, vn, vg;
        } cur, nxt;
        auto fetch1 = [&](int c, Rec1& r) {
            const int64_t rec = record(c, min(16 * wave + n, c1 - 1 - c0 - 64 * c));
            TL::load(p.k_codes + rec * Q::CW + Q::word0(qk), p.k_signs + rec * MW, PER, lane, r.raw);
            r.nu = p.k_norm[rec];
            r.gm = M > 0 ? (p.k_mu ? k_head : p.k_rnorm[rec]) : 0.f;
            r.vn = p.v_norm[rec];
            r.vg = M > 0 ? (p.v_mu ? v_head : p.v_rnorm[rec]) : 0.f;
        };
        if (c0 + 16 * wave < c1) fetch1(0, cur);
        for (int c = 0; c < nch; ++c) {
            const int key0 = c0 + 64 * c + 16 * wave;
            if (key0 + 64 < c1) fetch1(c + 1, nxt);  // the same for the whole wave
            float a[NRT];
            if (key0 < c1) {  // the same for the whole wave
                const bool valid = key0 + n < c1;
                double lg[NRT];
                tl.compute(cur.raw, cur.gm, PER, lane, lg);
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt)
                    a[rt] = valid ? (float)((double)p.scale * (double)cur.nu * lg[rt]) : -INFINITY;
                if (valid) {
                    numax = fmaxf(numax, cur.vn);
                    ngmax = fmaxf(ngmax, cur.vn * cur.vg);
                }
            } else {
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt) a[rt] = -INFINITY;
            }
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                lgs[((wave * NCH + c) * NRT + rt) * 64 + lane] = a[rt];
                mx[rt] = fmaxf(mx[rt], a[rt]);
            }
            cur = nxt;
        }
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        mx[rt] = max16(mx[rt]);
        if (n == 0) red[(wave * NRT + rt) * 4 + qk] = mx[rt];
    }
    numax = max64(numax);
    ngmax = max64(ngmax);
    if (lane == 0) {
        red[16 * NRT + wave] = numax;
        red[16 * NRT + 4 + wave] = ngmax;
    }
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        float v = red[rt * 4 + qk];
#pragma unroll
        for (int w = 1; w < 4; ++w) v = fmaxf(v, red[(w * NRT + rt) * 4 + qk]);
        mx[rt] = v;
    }
    numax = fmaxf(fmaxf(red[16 * NRT], red[16 * NRT + 1]), fmaxf(red[16 * NRT + 2], red[16 * NRT + 3]));
    ngmax = fmaxf(fmaxf(red[16 * NRT + 4], red[16 * NRT + 5]), fmaxf(red[16 * NRT + 6], red[16 * NRT + 7]));
    // weights: w = p nu <= max nu, w gamma <= max nu gamma (p <= 1)
    const int sw = dev::fixed_shift(numax);
    const int sz = dev::fixed_shift(ngmax);
    // 2^sw, 2^sz as floats (w * 2^sw < 2^26 is exact; tiny norms clamp the exponent)
    const float wscale = ldexpf(1.0f, min(sw, 126));
    const float zscale = ldexpf(1.0f, min(sz, 126));

    // ---------------- pass 2: weighted value sums on the matrix cores
    float lsum[NRT];
    intx4 accy[NRT][CBW][3];
    intx4 accz[NRT][ZBW > 0 ? ZBW : 1];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        lsum[rt] = 0.f;
#pragma unroll
        for (int j = 0; j < CBW; ++j)
#pragma unroll
            for (int bb = 0; bb < 3; ++bb) accy[rt][j][bb] = intx4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < (ZBW > 0 ? ZBW : 1); ++j) accz[rt][j] = intx4{0, 0, 0, 0};
    }
    uint32_t tdv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) tdv[i] = p.tdig_v[i];
    const int row = 16 * wave + n;  // this lane's key row within a 64-key chunk

    // value record of the lane's key (a clamped, valid record past the end;
    // its weight is zero), loaded one chunk ahead
    struct Rec2 {
        uint32_t W[Q::NW];
        uint32_t sg;  // the sign word holding sketch rows [qk*PER, (qk+1)*PER)
        float vn, vg;
    } vcur, vnxt;
    auto fetch2 = [&](int c, Rec2& r) {
        const int64_t rec = record(c, min(row, c1 - 1 - c0 - 64 * c));
        Q::load(p.v_codes + rec * Q::CW + Q::word0(qk), qk, r.W);
        r.sg = M > 0 ? p.v_signs[rec * MW + ((qk * PER) >> 5)] : 0u;
        r.vn = p.v_norm[rec];
        r.vg = M > 0 ? (p.v_mu ? v_head : p.v_rnorm[rec]) : 0.f;
    };
    fetch2(0, vcur);
    for (int c = 0; c < nch; ++c) {
        if (c + 1 < nch) fetch2(c + 1, vnxt);
        const uint32_t* W = vcur.W;
        const float vn = vcur.vn;
        const float vg = vcur.vg;
        // weights in fixed point, digits in the A-operand rows 4 qk + digit
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const float a = lgs[((wave * NCH + c) * NRT + rt) * 64 + lane];
            const float pj = __expf(a - mx[rt]);  // exp(-inf) = 0 past the end
            lsum[rt] += pj;
            const float w = pj * vn;
            const uint32_t Wi = (uint32_t)rintf(w * wscale);
            *reinterpret_cast<uint32_t*>(wd + ((0 * NRT + rt) * 64 + row) * 16 + 4 * qk) = digits4_unsigned(Wi);
            if constexpr (M > 0) {
                const uint32_t Zi = (uint32_t)rintf((w * vg) * zscale);
                *reinterpret_cast<uint32_t*>(wd + ((1 * NRT + rt) * 64 + row) * 16 + 4 * qk) = digits4_unsigned(Zi);
            }
        }
        // level digits of the lane's coordinate quarter: column blocks qk*CBW + j
#pragma unroll
        for (int j = 0; j < CBW; ++j) {
            uint32_t sel[4];
#pragma unroll
            for (int sg = 0; sg < 4; ++sg) sel[sg] = Q::sel(W, 4 * j + sg, qk);
#pragma unroll
            for (int bb = 0; bb < 3; ++bb) {
                intx4 v;
#pragma unroll
                for (int sg = 0; sg < 4; ++sg) v[sg] = (int)dev::lut4(tdv, bb, sel[sg]);
                *reinterpret_cast<intx4*>(vy + ((bb * NCB + qk * CBW + j) * 64 + row) * 16) = v;
            }
        }
        // sign bits of sketch rows [qk*PER, (qk+1)*PER) as +-1 bytes
        if constexpr (M > 0) {
            if constexpr (PER >= 16) {
#pragma unroll
                for (int k = 0; k < PER / 16; ++k) {
                    const int bit0 = qk * PER + 16 * k;
                    const uint32_t x = vcur.sg >> (bit0 & 31);
                    intx4 v;
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) v[s4] = (int)dev::spread4_pm(x >> (4 * s4));
                    *reinterpret_cast<intx4*>(vz + ((bit0 >> 4) * 64 + row) * 16) = v;
                }
            } else {
                const int bit0 = qk * PER;
                const uint32_t x = vcur.sg >> (bit0 & 31);
                intx2 v;
                v[0] = (int)dev::spread4_pm(x);
                v[1] = (int)dev::spread4_pm(x >> 4);
                *reinterpret_cast<intx2*>(vz + ((bit0 >> 4) * 64 + row) * 16 + (bit0 & 15)) = v;
            }
        }
        __syncthreads();
        intx4 aw[NRT], az[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            aw[rt] = tr_operand(wd + (0 * NRT + rt) * 1024, lane);
            if constexpr (M > 0) az[rt] = tr_operand(wd + (1 * NRT + rt) * 1024, lane);
        }
#pragma unroll
        for (int j = 0; j < CBW; ++j) {
            const int cb = wave * CBW + j;
#pragma unroll
            for (int bb = 0; bb < 3; ++bb) {
                const intx4 bv = tr_operand(vy + (bb * NCB + cb) * 1024, lane);
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt)
                    accy[rt][j][bb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aw[rt], bv, accy[rt][j][bb], 0, 0, 0);
            }
        }
        if constexpr (M > 0) {
#pragma unroll
            for (int j = 0; j < ZBW; ++j) {
                const int cs = wave + 4 * j;
                if (cs < NZB) {
                    const intx4 bz = tr_operand(vz + cs * 1024, lane);
#pragma unroll
                    for (int rt = 0; rt < NRT; ++rt)
                        accz[rt][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(az[rt], bz, accz[rt][j], 0, 0, 0);
                }
            }
        }
        __syncthreads();
        vcur = vnxt;
    }

    // ---------------- partial results of the split
    // l per query: lanes of one query hold disjoint keys; then across waves
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        lsum[rt] = sum16(lsum[rt]);
        if (n == 0) red[(wave * NRT + rt) * 4 + qk] = lsum[rt];
    }
    __syncthreads();
    const double yscale = ldexp(1.0, -(sw + p.shift_v));
    const double zs = ldexp(1.0, -sz);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        const int g = gq0 + 4 * rt + qk;  // lane's query in the MFMA result rows 4 qk .. 4 qk + 3
        if (g >= G) continue;
        float* dst = p.part + ((rowbase + g) * p.nsplit + split) * width;
        if (wave == 0 && n == 0) {
            dst[0] = mx[rt];
            dst[1] = (red[rt * 4 + qk] + red[(NRT + rt) * 4 + qk]) + (red[(2 * NRT + rt) * 4 + qk] + red[(3 * NRT + rt) * 4 + qk]);
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
            for (int j = 0; j < ZBW; ++j) {
                const int cs = wave + 4 * j;
                if (cs < NZB) dst[2 + D + 16 * cs + n] = (float)(digit_rows(accz[rt][j]) * zs);
            }
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
    for (int i = 0; i < 8; ++i) {
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
