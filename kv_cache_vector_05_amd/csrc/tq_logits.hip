// Attention-logit scan from packed keys on the integer matrix cores
// (tambur post: logits straight from quantised keys; iaemfoco post, "TurboQuant:
// Uma Nova Abordagem" and itstec post, "Por dentro do processo de compressao
// KV": the unbiased one-bit QJL correction):
//     logit = nu ( <q', t[c]> + sqrt(pi/2)/m * gamma * <s, z> ),  q' = Pi RoPE(q), s = S q',
// or, with the sign correction (TurboESM summary, technical section 2),
//     logit = nu ( <q', t[c]> + mu_head <q', z> )  (S = I, so s = q').
//
// Exact integer formulation.  Every float that enters a product is turned
// into a fixed-point integer split into balanced int8 digits: q' and s once
// per query (here, in the query-prep kernel) as 28 bits in four base-128
// digits, the levels t_k once per codebook (on the host) as 24 bits in three
// base-256 digits, each with its own power-of-two scale.  The products of digits are summed exactly in int32 by
// v_mfma_i32_16x16x64_i8, the digit sums are combined in int32 and fp64 and
// only the final value is rounded to fp32; the residual error is the
// rounding of q', s (2^-27 of their largest entry) and t (2^-24 of the
// largest level) to fixed point, below an fp32 dot product's own error.
//
// MFMA shape: rows = (query, digit of q') - four digits of four queries fill
// the 16 rows, so a GQA group of 4 wastes nothing - columns = 16 keys, K = 64
// coordinates.  Lane l of the wave owns key l % 16 and the coordinate quarter
// l / 16 ([q*d/4, (q+1)*d/4)), which for d = 128, b = 3 is exactly three whole
// code words; its 16 K-slots per MFMA are 16 consecutive coordinates.  The B
// operand (digit b of t[c] for the 16 coordinates) is built with one v_perm
// per 4 coordinates from an 8-byte digit table.  After the MFMAs, lane l holds
// all 12 digit products of (query l/16, key l%16): rows 4(l/16)+r = digit r.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

__device__ __forceinline__ int clamp_len2(const int32_t* seq_len, int b, int L_cap) {
    int s = seq_len[b];
    return s < 0 ? 0 : (s > L_cap ? L_cap : s);
}

// block-wide max of |v| and sum of v over 256 threads
__device__ __forceinline__ void block_absmax_sum(float v, float* red, float* amax, float* sum) {
    float a = fabsf(v), s = v;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        a = fmaxf(a, __shfl_xor(a, o));
        s += __shfl_xor(s, o);
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
        red[threadIdx.x >> 6] = a;
        red[4 + (threadIdx.x >> 6)] = s;
    }
    __syncthreads();
    *amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    *sum = (red[4] + red[5]) + (red[6] + red[7]);
}

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
    int32_t norot;    // Pi = I: q' = RoPE(q)
    int32_t s_ident;  // S = I (sign correction): s = q'
    const int32_t* seq_len;
    const int32_t* q_pos;
    const float* rope_cos;
    const float* rope_sin;
    const float* sigma;
    const float* sketch;
    float* qp;       // [rows][D]    q' (fp32)
    float* s;        // [rows][m]    s = S q' (fp32)
    int8_t* qd;      // [rows*4][D]  digits of q' (digit rows 4*row + a)
    int8_t* sd;      // [rows*4][sdw] digits of s in MFMA slot order
    float* scale;    // [rows][3]    shift(q'), shift(s), sum of the fixed-point s values
};

// One workgroup per query head: RoPE, sign flips, Walsh-Hadamard, 1/sqrt(d),
// s = S q', then the fixed-point digit rows.
template <int D>
__global__ __launch_bounds__(256) void qprep_digits_kernel(QDig p) {
    __shared__ float xs[D];
    __shared__ float sv[D];
    __shared__ float red[8];
    const int t = threadIdx.x;
    const int64_t bh = blockIdx.x;
    const int b = (int)(bh / p.Hq);
    if (t < D) {
        xs[t] = p.bf16 ? __uint_as_float((uint32_t) static_cast<const uint16_t*>(p.q)[bh * D + t] << 16)
                       : static_cast<const float*>(p.q)[bh * D + t];
    }
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
    if (!p.norot) {
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
    }
    const float inv = p.norot ? 1.0f : 1.0f / sqrtf((float)D);
    float qv = 0.f;
    if (t < D) {
        qv = xs[t] * inv;
        xs[t] = qv;
        p.qp[bh * D + t] = qv;
    }
    __syncthreads();
    float sval = 0.f;
    if (t < p.m) {
        if (p.s_ident) {
            sval = xs[t];
        } else {
            const float* row = p.sketch + (int64_t)t * D;
            for (int i = 0; i < D; ++i) sval = fmaf(row[i], xs[i], sval);
        }
        sv[t] = sval;
        p.s[bh * p.m + t] = sval;
    }
    float qmax, qsum, smax, ssum;
    block_absmax_sum(qv, red, &qmax, &qsum);
    block_absmax_sum(sval, red, &smax, &ssum);
    const int shq = fixed_shift(qmax);
    const int shs = fixed_shift(smax);
    if (t < D) {
        int8_t d[4];
        digits4(to_fixed(qv, shq), d);
        for (int a = 0; a < 4; ++a) p.qd[(bh * 4 + a) * D + t] = d[a];
    }
    // sketch digits in MFMA slot order: byte (qk*ncs + cs)*16 + j holds
    // sketch row qk*(m/4) + 16*cs + j (zero where that slot is past m/4)
    long long sfix = 0;
    if (t < p.m) sfix = to_fixed(sval, shs);
    __syncthreads();
    if (p.m) {
        for (int off = t; off < p.sdw; off += blockDim.x) {
            const int qk = off / (16 * p.ncs), rem = off % (16 * p.ncs);
            const int cs = rem / 16, j = rem % 16;
            const int l = qk * (p.m / 4) + 16 * cs + j;
            int8_t d[4] = {0, 0, 0, 0};
            if (16 * cs + j < p.m / 4) digits4(to_fixed(sv[l], shs), d);
            for (int a = 0; a < 4; ++a) p.sd[(bh * 4 + a) * p.sdw + off] = d[a];
        }
    }
    // sum of the fixed-point s values (exact integer), for sum_l s_l z_l = 2 sum_l s_l bit_l - sum_l s_l
    double sf = (double)sfix;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sf += __shfl_xor(sf, o);
    __syncthreads();
    __shared__ double dred[4];
    if ((t & 63) == 0) dred[t >> 6] = sf;
    __syncthreads();
    if (t == 0) {
        p.scale[bh * 3 + 0] = (float)shq;  // shifts are small integers, exact in fp32
        p.scale[bh * 3 + 1] = (float)shs;
        p.scale[bh * 3 + 2] = (float)ldexp((dred[0] + dred[1]) + (dred[2] + dred[3]), -shs);
    }
}

struct LogM {
    const int8_t* qd;
    const int8_t* sd;
    const float* scale;
    const float* norm;
    const float* rnorm;
    const uint32_t* codes;
    const uint32_t* signs;
    const int32_t* seq_len;
    int32_t Hq, h_kv, L_cap, m, sdw, ngroups, tiles_per_wave;
    int32_t k0, klen;
    float* out;
    int64_t ld;
    int32_t col0;
    uint32_t tdig[8];
    int32_t lvl_shift;
    double cq;           // scale of the correction term
    const float* mu;     // sign correction: mu per KV head (stride mu_stride), else nullptr
    int32_t mu_stride;
    // paged records: page table [B][max_pages] of pages of page_size slots
    // (a multiple of 64); entries are clamped into [0, n_pages)
    const int32_t* pages;
    int32_t page_size, max_pages;
    int64_t n_pages;
    dev::FastDiv div_page;
};

// Record index of key `key` of (sequence b, KV head kh) through the page table
// (key0: a wave-uniform key of the same page, from which the page is found).
__device__ __forceinline__ int64_t paged_record(const int32_t* pages, int32_t page_size, int32_t max_pages,
                                                int64_t n_pages, const dev::FastDiv& div_page, int h_kv, int b, int kh,
                                                int key) {
    const uint32_t j = div_page.div((uint32_t)key);
    int64_t pg = pages[(int64_t)b * max_pages + j];
    pg = pg < 0 ? 0 : (pg >= n_pages ? n_pages - 1 : pg);
    return (pg * h_kv + kh) * page_size + (key - (int64_t)j * page_size);
}

template <int D, int BITS, int NRT, int NCS, bool PAGED>
__global__ __launch_bounds__(256) void logits_mfma_kernel(LogM p) {
    using T = dev::TileLogit<D, BITS, NRT, NCS>;
    using Q = typename T::Q;
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

    T tl;
    tl.init(p.qd, p.sd, p.scale, p.sdw, p.cq, rowbase, gq0, G, p.tdig, p.lvl_shift, lane);
    // correction weight: gamma per key (QJL sketch) or the KV head's mu
    const bool g_per_key = p.mu == nullptr;
    const float g_head = g_per_key ? 0.0f : p.mu[kh * p.mu_stride];

    const int sl = clamp_len2(p.seq_len, b, p.L_cap);
    const int kend = min(sl, p.k0 + p.klen);
    const int kbeg = p.k0 + (blockIdx.y * (blockDim.x >> 6) + wave) * p.tiles_per_wave * 16;
    // (tile counts are wave-uniform: kept in scalar registers for scalar branches)
    const int ntile = __builtin_amdgcn_readfirstlane(min(p.tiles_per_wave, (kend - kbeg + 15) / 16));
    if (ntile <= 0) return;
    const int nfull = __builtin_amdgcn_readfirstlane(min(p.tiles_per_wave, (kend - kbeg) / 16));
    const int mw = p.m >> 5;
    const int per = p.m >> 2;  // sketch rows per lane group (8, 16, 32, ...)
    // per-lane pointers at the lane's key of the wave's first tile; a tile
    // advances them by 16 records
    const int64_t rec0 = bk * p.L_cap + kbeg + n;
    const uint32_t* cptr = p.codes + rec0 * Q::CW + Q::word0(qk);
    const uint32_t* sptr = p.signs + rec0 * mw;
    const float* nptr = p.norm + rec0;
    const float* gptr = p.rnorm + rec0;
    const int g_lane = gq0 + qk;  // the lane's query in row tile 0
    float* optr = p.out + (rowbase + g_lane) * p.ld + (kbeg + n - p.col0);
    const int64_t ort = 4 * p.ld;  // next row tile
    const bool rows_full = gq0 + 4 * NRT <= G;

    // Tiles go in pairs: both tiles' MFMAs are issued before either is
    // combined, so one tile's operand building and digit combination overlap
    // the other's matrix work.  The records of the next pair are loaded while
    // a pair computes (four register slots, the loop unrolled by two pairs so
    // that no slot is copied).  Full tiles take a path without key guards.
    typename T::Raw rs[4];
    float nus[4], gms[4];
    auto fetch = [&](int tile, int slot) {
        if constexpr (PAGED) {
            // a full tile's 16 keys share one page (wave-uniform lookup); a
            // partial last tile reads the record of its last valid key instead
            int64_t rec;
            if (tile < nfull) {
                const int key0 = __builtin_amdgcn_readfirstlane(kbeg + tile * 16);
                rec = paged_record(p.pages, p.page_size, p.max_pages, p.n_pages, p.div_page, p.h_kv, b, kh, key0) + n;
            } else {
                const int key = min(kbeg + tile * 16 + n, kend - 1);
                rec = paged_record(p.pages, p.page_size, p.max_pages, p.n_pages, p.div_page, p.h_kv, b, kh, key);
            }
            T::load(p.codes + rec * Q::CW + Q::word0(qk), p.signs + rec * mw, per, lane, rs[slot]);
            nus[slot] = p.norm[rec];
            gms[slot] = NCS > 0 ? (g_per_key ? p.rnorm[rec] : g_head) : 0.0f;
        } else if (tile < nfull) {  // uniform record offset
            const int off = tile * 16;
            T::load(cptr + off * Q::CW, sptr + off * mw, per, lane, rs[slot]);
            nus[slot] = nptr[off];
            gms[slot] = NCS > 0 ? (g_per_key ? gptr[off] : g_head) : 0.0f;
        } else {  // a partial last tile reads the record of its last valid key instead
            const int off = min(tile * 16, kend - 1 - kbeg - n);
            T::load(cptr + off * Q::CW, sptr + off * mw, per, lane, rs[slot]);
            nus[slot] = nptr[off];
            gms[slot] = NCS > 0 ? (g_per_key ? gptr[off] : g_head) : 0.0f;
        }
    };
    auto store = [&](int tile, int slot, const double* lg) {
        const bool ok = tile < nfull || kbeg + tile * 16 + n < kend;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const float v = (float)lg[rt] * nus[slot];
            if (rows_full && tile < nfull) optr[rt * ort + tile * 16] = v;
            else if (ok && g_lane + 4 * rt < G) optr[rt * ort + tile * 16] = v;
        }
    };
    auto pair = [&](int tile, int s0) {
        const int s2 = s0 ^ 2;
        if (tile + 2 < ntile) fetch(tile + 2, s2);
        if (tile + 3 < ntile) fetch(tile + 3, s2 + 1);
        typename T::Acc a0, a1;
        tl.mma(rs[s0], per, lane, a0);
        const bool two = tile + 1 < ntile;
        if (two) tl.mma(rs[s0 + 1], per, lane, a1);
        double lg[NRT];
        tl.finish(a0, gms[s0], lg);
        store(tile, s0, lg);
        if (two) {
            tl.finish(a1, gms[s0 + 1], lg);
            store(tile + 1, s0 + 1, lg);
        }
    };
    fetch(0, 0);
    if (ntile > 1) fetch(1, 1);
    for (int tile = 0; tile < ntile; tile += 4) {
        pair(tile, 0);
        if (tile + 2 < ntile) pair(tile + 2, 2);
    }
}

using LogMFn = void (*)(LogM);

template <int D, int BITS, int NRT, bool PG>
LogMFn pick_ncs(int m) {
    const int ncs = m == 0 ? 0 : std::max(1, m / 64);
    switch (ncs) {
        case 0: return logits_mfma_kernel<D, BITS, NRT, 0, PG>;
        case 1: return logits_mfma_kernel<D, BITS, NRT, 1, PG>;
        case 2: return logits_mfma_kernel<D, BITS, NRT, 2, PG>;
    }
    return nullptr;
}
template <int D, int BITS, bool PG>
LogMFn pick_nrt(int nrt, int m) {
    if (nrt == 1) return pick_ncs<D, BITS, 1, PG>(m);
    if (nrt == 2) return pick_ncs<D, BITS, 2, PG>(m);
    if (nrt == 4) return pick_ncs<D, BITS, 4, PG>(m);
    return nullptr;
}
template <int D, bool PG>
LogMFn pick_bits_m(int bits, int nrt, int m) {
    switch (bits) {
        case 1: return pick_nrt<D, 1, PG>(nrt, m);
        case 2: return pick_nrt<D, 2, PG>(nrt, m);
        case 3: return pick_nrt<D, 3, PG>(nrt, m);
    }
    return nullptr;
}

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// workgroups of 256 threads of kernel fn that fit on the device at once
int64_t resident_blocks(const void* fn) {
    static thread_local const void* last_fn = nullptr;
    static thread_local int64_t last = 0;
    if (fn == last_fn) return last;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0) != hipSuccess || per_cu < 1)
        return 1024;
    last_fn = fn;
    last = (int64_t)cus * per_cu;
    return last;
}

}  // namespace

bool logits_mfma_supported(const tq_codebook* ck) {
    return !ck->dense && ck->spec.block < 2 && ck->spec.bits <= 3 && (ck->spec.d == 64 || ck->spec.d == 128) && ck->spec.m <= 128;
}

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
    p.seq_len = a.seq_len;
    p.q_pos = a.q_pos;
    p.rope_cos = a.rope_cos;
    p.rope_sin = a.rope_sin;
    p.sigma = ck->dev.sigma;
    p.sketch = ck->dev.sketch;
    p.norot = no_rotation(ck) ? 1 : 0;
    p.s_ident = sign_corr(ck) ? 1 : 0;
    p.qp = q.qp;
    p.s = q.s;
    p.qd = q.qd;
    p.sd = q.sd;
    p.scale = q.scale;
    const unsigned grid = (unsigned)((int64_t)a.B * a.Hq);
    if (ck->spec.d == 64) hipLaunchKernelGGL(qprep_digits_kernel<64>, dim3(grid), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL(qprep_digits_kernel<128>, dim3(grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_logits_mfma(const tq_codebook* ck, const tq_packed& k, const AttnArgs& a, const QDigits& q,
                              int k0, int klen, float* out, int64_t ld, int col0, hipStream_t stream) {
    const int G = a.Hq / a.h_kv;
    const int nrt = G <= 4 ? 1 : (G <= 8 ? 2 : 4);
    const int ngroups = (G + 4 * nrt - 1) / (4 * nrt);
    LogMFn fn = nullptr;
    const bool paged = a.pages.table != nullptr;
    if (ck->spec.d == 64)
        fn = paged ? pick_bits_m<64, true>(ck->spec.bits, nrt, ck->spec.m) : pick_bits_m<64, false>(ck->spec.bits, nrt, ck->spec.m);
    else if (ck->spec.d == 128)
        fn = paged ? pick_bits_m<128, true>(ck->spec.bits, nrt, ck->spec.m) : pick_bits_m<128, false>(ck->spec.bits, nrt, ck->spec.m);
    if (!fn) return hipErrorInvalidValue;
    LogM p{};
    p.qd = q.qd;
    p.sd = q.sd;
    p.scale = q.scale;
    p.norm = k.norm;
    p.rnorm = k.rnorm;
    p.codes = k.codes;
    p.signs = k.signs;
    p.seq_len = a.seq_len;
    p.Hq = a.Hq;
    p.h_kv = a.h_kv;
    p.L_cap = a.L_cap;
    p.m = ck->spec.m;
    p.sdw = q.sdw;
    p.ngroups = ngroups;
    p.k0 = k0;
    p.klen = klen;
    p.out = out;
    p.ld = ld;
    p.col0 = col0;
    for (int i = 0; i < 8; ++i) p.tdig[i] = ck->lvl_digits[i];
    p.lvl_shift = ck->lvl_shift;
    p.cq = corr_scale(ck);
    const MuRef mr = mu_ref(ck);
    p.mu = mr.ptr;
    p.mu_stride = mr.stride;
    p.pages = a.pages.table;
    p.page_size = a.pages.size;
    p.max_pages = a.pages.max_pages;
    p.n_pages = a.pages.n_pages;
    p.div_page = dev::FastDiv((uint32_t)(a.pages.size > 0 ? a.pages.size : 1));
    // Size the work per wave so that the whole grid is resident at once (one
    // round of workgroups, no partly idle last round).
    const int64_t gx = (int64_t)a.B * a.h_kv * ngroups;
    const int64_t tiles_row = (klen + 15) / 16;  // 16-key tiles per (sequence, KV head)
    if (gx == 0 || tiles_row == 0) return hipSuccess;
    const int64_t resident = resident_blocks((const void*)fn);
    const int64_t gy_want = std::max<int64_t>(1, (resident + gx - 1) / gx);
    p.tiles_per_wave = (int)std::max<int64_t>(1, (tiles_row + 4 * gy_want - 1) / (4 * gy_want));
    const int64_t gy = (tiles_row + 4 * (int64_t)p.tiles_per_wave - 1) / (4 * (int64_t)p.tiles_per_wave);
    hipLaunchKernelGGL(fn, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace tq
