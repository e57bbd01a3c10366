// Attention-logit scan from packed keys on the integer matrix cores
// (tambur post: logits straight from quantised keys; iaemfoco post,
// "TurboQuant: Uma Nova Abordagem" and itstec post, "Por dentro do processo de
// compressao KV": the one-bit QJL correction):
//     logit = nu ( <q', t[c]> + sqrt(pi/2)/m * gamma * <s, z> ),  q' = Pi RoPE(q), s = S q',
// or, with the sign correction (TurboESM summary, technical section 2),
//     logit = nu ( <q', t[c]> + mu_head <q', z> )  (S = I, so s = q').
//
// Exact integer arithmetic on v_mfma_i32_16x16x64_i8: rows = (query, digit
// of q'), columns = 16 keys, K = 64 coordinates.  The queries arrive prepared
// (tq_qprep.hip: q' and s as four balanced base-128 digits with one scale per
// query); the levels' three base-256 digits come from the packed codes by one
// v_perm per four coordinates; the sign bits become 0/1 bytes through a
// 256-entry LDS table.  The digit sums are exact; the digit rows pair
// exactly in int32 and the rest of the combination runs in fp32.  Lane l
// owns key l % 16 and coordinate quarter l / 16, and holds the logit of
// (query l / 16, key l % 16) of each four-query row tile.
//
// One workgroup serves one KV head of one sequence, up to 4 NRT of its query
// heads and a contiguous run of keys, sized so that the whole grid is
// resident at once: eight waves when it prepares its four queries itself
// (one row tile; the preparation runs once per workgroup, on four of the
// waves), four waves reading prepared queries otherwise.  Records are read
// with buffer loads whose per-tile advance is a scalar offset (no vector
// instructions on addresses); every load is unconditional, so each wave keeps
// its next eight (four) tiles of records in flight behind the one it
// computes.
#include <hip/hip_runtime.h>

#include <type_traits>

#include <algorithm>
#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

using dev::intx4;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRsrcWord3 = 0x00020000;  // buffer resource word 3 for gfx9: 32-bit elements, no swizzle
// cache policy of the logit stores: nt (streaming; each logit is written
// once).  The record loads keep the default policy: streaming loads measured
// slower.
constexpr int kStream = 2;

// buffer resource over [base, base + bytes); loads past the end return 0
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3);
}

struct ScanArgs {
    dev::PrepIn prep;       // one row tile: the queries and the tables their preparation reads
    const int32_t* q_pos;   // queries' RoPE positions (nullptr: seq_len)
    const int8_t* qd;       // several row tiles: queries prepared by tq_qprep.hip (digit rows of q')
    const int8_t* sd;       // digit rows of s in MFMA slot order
    const float* scale;     // per query: shift(q'), shift(s), sum of the fixed-point s
    int32_t sdw;
    const int32_t* seq_len;
    const float* norm;
    const float* rnorm;
    const uint32_t* codes;
    const uint32_t* signs;
    int64_t cap;            // records in each plane
    int32_t Hq, h_kv, L_cap, m, ngroups, tiles_per_wave, k0, klen;
    float* out;
    int64_t ld;
    int32_t col0;
    uint32_t tdig[16];
    int32_t lvl_shift;
    double cq;              // scale of the correction term
    const float* mu;        // sign correction: mu per KV head (stride mu_stride)
    int32_t mu_stride;
    const int32_t* pages;   // paged records: [B][max_pages], pages of page_size slots
    int32_t page_size, max_pages;
    int64_t n_pages;
    dev::FastDiv div_page;
};

// waves per workgroup: a single row tile prepares its queries in the kernel,
// on four of the waves, so the workgroup is wider than four waves (the
// preparation is repeated once per workgroup); eight waves, two workgroups
// per CU, measured faster than one sixteen-wave workgroup.  More row tiles
// read prepared queries and keep four waves.
constexpr int kFusedWaves = 8;
// one row tile always; two without a sketch (with one, the eight rows'
// sketch product and the second tile's operands cost more than the separate
// preparation they save)
constexpr bool scan_fused(int nrt, int m) { return nrt == 1 || (nrt == 2 && m == 0); }
template <int NRT, int M>
constexpr int scan_waves() {
    return scan_fused(NRT, M) ? kFusedWaves : 4;
}
// tiles of records each wave keeps in flight behind the one it computes: the
// wide workgroup runs at four waves per SIMD whatever its register count, so
// one row tile takes twice the depth (the bytes in flight set the streaming
// rate); two row tiles, and paged 4-bit records, need the registers
constexpr int scan_depth(int nrt, int bits, bool paged) { return nrt == 1 && !(paged && bits == 4) ? 8 : 4; }

template <int D, int BITS, int NRT, int M, bool PAGED>
__global__ __launch_bounds__((64 * scan_waves<NRT, M>())) void scan_kernel(ScanArgs p) {
    using Q = dev::Quarter<D, BITS>;
    constexpr int R = 4 * NRT;       // query rows of the workgroup
    constexpr int NC = Q::LPG / 16;  // K = 64 chunks over the lane's coordinates
    constexpr bool FUSE = scan_fused(NRT, M);
    constexpr int ST = FUSE && scan_waves<NRT, M>() >= 8 ? 512 : 256;  // threads of the sketch product
    using PL = dev::PrepLds<D, M, R, ST>;
    constexpr int NCS = PL::NCS;     // K = 64 chunks of the sketch product
    // The workgroup prepares its queries itself (one row tile, or two
    // without a sketch); otherwise it reads the queries prepared beforehand.
    __shared__ u32x2 stab[256];      // bits of a byte -> eight 0/1 bytes
    __shared__ std::conditional_t<FUSE, PL, char> prep;  // the workgroup's prepared queries

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: scalar addresses
    const int n = lane & 15;
    const int qk = lane >> 4;
    const int grp = blockIdx.x % p.ngroups;
    const int64_t bk = blockIdx.x / p.ngroups;
    const int b = (int)(bk / p.h_kv);
    const int kh = (int)(bk % p.h_kv);
    const int G = p.Hq / p.h_kv;
    const int64_t rowbase = (int64_t)b * p.Hq + (int64_t)kh * G;
    const int gq0 = grp * R;

    const int sl = dev::clamp_len(p.seq_len, b, p.L_cap);
    const int kend = min(sl, p.k0 + p.klen);
    // a workgroup without keys leaves at once (before any barrier)
    constexpr int NWV = scan_waves<NRT, M>();
    if (p.k0 + (int)blockIdx.y * NWV * p.tiles_per_wave * 16 >= kend) return;
    const int kbeg = p.k0 + ((int)blockIdx.y * NWV + wave) * p.tiles_per_wave * 16;
    const int ntile = __builtin_amdgcn_readfirstlane(max(0, min(p.tiles_per_wave, (kend - kbeg + 15) / 16)));
    const int nfull = __builtin_amdgcn_readfirstlane(max(0, min(p.tiles_per_wave, (kend - kbeg) / 16)));
    const int mw = p.m >> 5;
    const int per = p.m >> 2;  // sketch rows per lane group: 8, 16 or 32

    // ---- record loads (per lane: its key's quarter of the code words, the
    // sign word holding its sketch rows, nu, gamma)
    constexpr int CW = Q::CW;
    const uint32_t vo_c = (uint32_t)(n * CW + Q::word0(qk)) * 4u;
    const uint32_t vo_s = (uint32_t)(n * mw + ((qk * per) >> 5)) * 4u;
    const uint32_t vo_n = (uint32_t)n * 4u;
    const bool g_per_key = p.mu == nullptr;
    const float g_head = g_per_key ? 0.0f : p.mu[kh * p.mu_stride];
    const int64_t rec_w = bk * p.L_cap + kbeg;  // contiguous records: the wave's first key
    __amdgpu_buffer_rsrc_t rc, rs_, rn, rg;
    if constexpr (!PAGED) {
        rc = make_rsrc(p.codes + rec_w * CW, (p.cap - rec_w) * CW * 4);
        rs_ = make_rsrc(p.signs + rec_w * mw, (p.cap - rec_w) * mw * 4);
        rn = make_rsrc(p.norm + rec_w, (p.cap - rec_w) * 4);
        rg = make_rsrc(g_per_key ? p.rnorm + rec_w : nullptr, g_per_key ? (p.cap - rec_w) * 4 : 0);
    }
    struct Raw {
        uint32_t W[Q::NW];
        uint32_t sg;
        float nu, gm;
        int64_t rec;  // paged: the tile's first record
    };
    // code and sign words of a tile (and, for paged records, its page)
    auto fetch_codes = [&](int tile, Raw& r) {
        uint32_t so_c, so_s;
        if constexpr (PAGED) {
            // a 16-key tile lies in one page (pages hold a multiple of 64 slots)
            const int key0 = kbeg + tile * 16;
            const uint32_t j = p.div_page.div((uint32_t)key0);
            int64_t pg = p.pages[(int64_t)b * p.max_pages + j];
            pg = pg < 0 ? 0 : (pg >= p.n_pages ? p.n_pages - 1 : pg);
            r.rec = (pg * p.h_kv + kh) * p.page_size + (key0 - (int64_t)j * p.page_size);
            rc = make_rsrc(p.codes + r.rec * CW, (p.cap - r.rec) * CW * 4);
            rs_ = make_rsrc(p.signs + r.rec * mw, (p.cap - r.rec) * mw * 4);
            so_c = so_s = 0;
        } else {
            so_c = (uint32_t)tile * 16u * CW * 4u;
            so_s = (uint32_t)tile * 16u * (uint32_t)mw * 4u;
        }
        if constexpr (Q::NW == 3) {
            const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rc, vo_c, so_c, 0);
            r.W[0] = v.x;
            r.W[1] = v.y;
            r.W[2] = v.z;
        } else if constexpr (Q::NW == 4 && Q::ALIGNED) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, vo_c, so_c, 0);
            r.W[0] = v.x;
            r.W[1] = v.y;
            r.W[2] = v.z;
            r.W[3] = v.w;
        } else if constexpr (Q::NW == 2 && Q::ALIGNED) {
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rc, vo_c, so_c, 0);
            r.W[0] = v.x;
            r.W[1] = v.y;
        } else if constexpr (Q::ALIGNED) {
#pragma unroll
            for (int i = 0; i < Q::NW; ++i) r.W[i] = __builtin_amdgcn_raw_buffer_load_b32(rc, vo_c + 4u * i, so_c, 0);
        } else {
            // the quarter straddles words: NW words from word0, the last clamped
            // into the record, shifted into place
            const int w0 = Q::word0(qk);
#pragma unroll
            for (int i = 0; i < Q::NW; ++i)
                r.W[i] = __builtin_amdgcn_raw_buffer_load_b32(rc, (uint32_t)(n * CW + w0 + min(i, CW - 1 - w0)) * 4u,
                                                              so_c, 0);
            const int sh = (Q::BPG * qk) & 31;
#pragma unroll
            for (int i = 0; i + 1 < Q::NW; ++i) r.W[i] = __builtin_amdgcn_alignbit(r.W[i + 1], r.W[i], sh);
        }
        r.sg = NCS > 0 ? __builtin_amdgcn_raw_buffer_load_b32(rs_, vo_s, so_s, 0) : 0u;
    };
    // nu and gamma of a tile (loaded after the tile's slot has been combined)
    auto fetch_scalars = [&](int tile, Raw& r) {
        uint32_t so_n;
        if constexpr (PAGED) {
            rn = make_rsrc(p.norm + r.rec, (p.cap - r.rec) * 4);
            rg = make_rsrc(g_per_key ? p.rnorm + r.rec : nullptr, g_per_key ? (p.cap - r.rec) * 4 : 0);
            so_n = 0;
        } else {
            so_n = (uint32_t)tile * 64u;
        }
        r.nu = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rn, vo_n, so_n, 0));
        // gamma per key, or the head's mu (the load then reads zeros)
        if constexpr (NCS > 0) {
            // an add rather than a select keeps the load unconditional
            r.gm = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, vo_n, so_n, 0)) + g_head;
        } else {
            r.gm = g_head;
        }
    };
    // ---- query preparation: every workgroup of a (sequence, KV head) row
    // tile prepares its rows itself (rows past the group repeat the last
    // query and are never stored).  Its loads go first, then the first
    // records: loads complete in order, so the preparation waits for its own
    // loads only and computes while those records are in flight.
    dev::Prep<D, M, FUSE ? R : 1, ST> pr;
    intx4 aq[NRT][NC];
    intx4 as[NRT][NCS > 0 ? NCS : 1];
    float sc[NRT][3];
    if constexpr (FUSE) {
        pr.load(p.prep, [&](int r) { return rowbase + min(gq0 + r, G - 1); },
                dev::query_pos(p.q_pos, p.seq_len, b, p.L_cap));
    } else {
        // A rows (query 4rt + (lane&15)/4, digit lane&3; a row past the
        // group repeats the last query and is never stored) and the scales of
        // the lane's output query 4rt + qk
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const int64_t drow = (rowbase + min(gq0 + 4 * rt + ((lane & 15) >> 2), G - 1)) * 4 + (lane & 3);
#pragma unroll
            for (int c = 0; c < NC; ++c)
                aq[rt][c] = *reinterpret_cast<const intx4*>(p.qd + drow * D + qk * Q::LPG + 16 * c);
#pragma unroll
            for (int cs = 0; cs < NCS; ++cs)
                as[rt][cs] = *reinterpret_cast<const intx4*>(p.sd + drow * p.sdw + (qk * NCS + cs) * 16);
            const int64_t orow = rowbase + min(gq0 + 4 * rt + qk, G - 1);
#pragma unroll
            for (int k = 0; k < 3; ++k) sc[rt][k] = p.scale[orow * 3 + k];
        }
    }
    // Every record fetch is unconditional: a tile past the wave's last
    // reloads the last one (a cache hit), so each loop step issues the same
    // loads and the waits for a tile's data leave the later tiles' in flight.
    const auto clampt = [&](int tile) { return max(0, min(tile, ntile - 1)); };
    // the first half of the tiles in flight are requested before the
    // preparation, the rest after it (all of them in flight across it would
    // raise the register peak)
    constexpr int PF = scan_depth(NRT, BITS, PAGED);
    Raw raw[PF];
#pragma unroll
    for (int i = 0; i < PF / 2; ++i) {
        fetch_codes(clampt(i), raw[i]);
        fetch_scalars(clampt(i), raw[i]);
    }
    if (t < 256) {
        const uint32_t v = (uint32_t)t;  // one table entry per thread of the first four waves
        stab[t] = u32x2{dev::spread4(v), dev::spread4(v >> 4)};
    }
    if constexpr (FUSE) {
        pr.compute(p.prep, prep);  // ends with a barrier (the sign table is ready too)
        // A rows (query (lane&15)/4, digit lane&3) and the scales of the
        // lane's output query qk
        const int r = (lane & 15) >> 2, a = lane & 3;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
            for (int c = 0; c < NC; ++c)
                aq[rt][c] = *reinterpret_cast<const intx4*>(&prep.qd[4 * rt + r][a][qk * Q::LPG + 16 * c]);
#pragma unroll
            for (int cs = 0; cs < NCS; ++cs)
                as[rt][cs] = *reinterpret_cast<const intx4*>(&prep.sd[4 * rt + r][a][(qk * NCS + cs) * 16]);
#pragma unroll
            for (int k = 0; k < 3; ++k) sc[rt][k] = prep.scl[4 * rt + qk][k];
        }
    } else {
        __syncthreads();
    }
#pragma unroll
    for (int i = PF / 2; i < PF; ++i) {
        fetch_codes(clampt(i), raw[i]);
        fetch_scalars(clampt(i), raw[i]);
    }
    // logit / nu = V 2^qe + gamma (Z 2^ze c2 - zc) (powers of two by ldexp,
    // so no scale leaves the fp32 range)
    int qe[NRT], ze[NRT];
    float c2[NRT], zc[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        qe[rt] = -p.lvl_shift - (int)sc[rt][0];
        const double c = NCS > 0 ? p.cq : 0.0;
        ze[rt] = -(int)sc[rt][1];
        c2[rt] = (float)(2.0 * c);
        zc[rt] = (float)(c * (double)sc[rt][2]);
    }
    uint32_t tdig[16];
#pragma unroll
    for (int i = 0; i < (BITS == 4 ? 16 : 8); ++i) tdig[i] = p.tdig[i];

    // ---- output: row (rowbase + gq0 + 4rt + qk), column key - col0
    const int g_lane = gq0 + qk;
    __amdgpu_buffer_rsrc_t ro = make_rsrc(p.out + (rowbase + gq0) * p.ld + (kbeg - p.col0), (int64_t)0xFFFFFFFF);
    const bool rows_full = gq0 + R <= G;

    struct Acc {
        intx4 y[NRT][3];
        intx4 z[NRT];
    };
    auto mma = [&](const Raw& r, Acc& A) {
        intx4 bd[NC][3];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int sg = 0; sg < 4; ++sg) {
                const uint32_t sel = Q::sel(r.W, 4 * c + sg, qk);
#pragma unroll
                for (int bb = 0; bb < 3; ++bb) bd[c][bb][sg] = (int)dev::lut<BITS>(tdig, bb, sel);
            }
        }
        intx4 bz[NCS > 0 ? NCS : 1];
        if constexpr (NCS > 0) {
#pragma unroll
            for (int cs = 0; cs < NCS; ++cs) {
                uint32_t x = r.sg >> ((qk * per + 16 * cs) & 31);
                if (per - 16 * cs < 16) x &= (1u << (per - 16 * cs)) - 1u;  // 8 rows: one byte
                const u32x2 lo = stab[x & 0xFFu];
                const u32x2 hi = stab[(x >> 8) & 0xFFu];
                bz[cs] = intx4{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
            }
        }
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
            for (int bb = 0; bb < 3; ++bb) A.y[rt][bb] = intx4{0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int bb = 0; bb < 3; ++bb)
                    A.y[rt][bb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[rt][c], bd[c][bb], A.y[rt][bb], 0, 0, 0);
            A.z[rt] = intx4{0, 0, 0, 0};
#pragma unroll
            for (int cs = 0; cs < NCS; ++cs)
                A.z[rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(as[rt][cs], bz[cs], A.z[rt], 0, 0, 0);
        }
    };
    // logit of (query 4rt + qk, key n) from its digit sums: y[b][a] is digit a
    // of q' (weight 128^(3-a)) times digit b of the level (weight 256^(2-b));
    // pairs of q' digits combine exactly in int32 (|y| <= 2^20)
    auto finish = [&](const Acc& A, float nu, float gm, int tile) {
        const bool key_ok = tile < nfull || kbeg + tile * 16 + n < kend;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            float V = 0.0f;
#pragma unroll
            for (int bb = 0; bb < 3; ++bb) V = fmaf(V, 256.0f, dev::digits4_f32(A.y[rt][bb]));
            float lg = ldexpf(V, qe[rt]);
            if constexpr (NCS > 0) {
                // sum_l s_l z_l = 2 sum_l s_l bit_l - sum_l s_l
                lg = fmaf(gm, fmaf(ldexpf(dev::digits4_f32(A.z[rt]), ze[rt]), c2[rt], -zc[rt]), lg);
            }
            const float v = lg * nu;
            if ((rows_full && tile < nfull) || (key_ok && g_lane + 4 * rt < G))
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ro,
                                                      (uint32_t)(((int64_t)(qk + 4 * rt) * p.ld + n) * 4),
                                                      (uint32_t)tile * 64u, kStream);
        }
    };
    // One tile per step: its MFMAs, then its slot refilled with the tile
    // PF ahead (code and sign words first, as soon as the MFMAs have read
    // them; nu and gamma once the tile is combined).  A tile past the
    // wave's last computes on a reloaded tile and stores nothing (the launch
    // gives waves multiples of PF tiles, so only the last wave of a row
    // does this).
    auto step = [&](int tile, int s0) {
        Acc a0;
        mma(raw[s0], a0);
        fetch_codes(clampt(tile + PF), raw[s0]);
        finish(a0, raw[s0].nu, raw[s0].gm, tile);
        fetch_scalars(clampt(tile + PF), raw[s0]);
    };
    for (int tile = 0; tile < ntile; tile += PF) {
#pragma unroll
        for (int i = 0; i < PF; ++i) step(tile + i, i);
    }
}

using ScanFn = void (*)(ScanArgs);

template <int D, int BITS, int NRT, bool PG>
ScanFn pick_ncs(int m) {
    switch (m) {
        case 0: return scan_kernel<D, BITS, NRT, 0, PG>;
        case 32: return scan_kernel<D, BITS, NRT, 32, PG>;
        case 64: return scan_kernel<D, BITS, NRT, 64, PG>;
        case 128: return scan_kernel<D, BITS, NRT, 128, PG>;
    }
    return nullptr;
}
template <int D, int BITS, bool PG>
ScanFn pick_nrt(int nrt, int m) {
    if (nrt == 1) return pick_ncs<D, BITS, 1, PG>(m);
    if (nrt == 2) return pick_ncs<D, BITS, 2, PG>(m);
    if (nrt == 4) return pick_ncs<D, BITS, 4, PG>(m);
    return nullptr;
}
template <int D, bool PG>
ScanFn pick_bits(int bits, int nrt, int m) {
    switch (bits) {
        case 1: return pick_nrt<D, 1, PG>(nrt, m);
        case 2: return pick_nrt<D, 2, PG>(nrt, m);
        case 3: return pick_nrt<D, 3, PG>(nrt, m);
        case 4: return pick_nrt<D, 4, PG>(nrt, m);
    }
    return nullptr;
}

// rounds of resident workgroups the launch is cut into
constexpr int kScanRounds = 1;

int64_t resident_blocks(const void* fn, int threads) {
    static thread_local const void* last_fn = nullptr;
    static thread_local int64_t last = 0;
    if (fn == last_fn) return last;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) != hipSuccess || per_cu < 1)
        return 1024 * 4 / (threads / 64);
    last_fn = fn;
    last = (int64_t)cus * per_cu;
    return last;
}

}  // namespace

bool scan_supported(const tq_codebook* ck) {
    const int m = ck->spec.m;
    return !ck->dense && ck->spec.block < 2 && ck->spec.bits <= 4 && (ck->spec.d == 64 || ck->spec.d == 128) &&
           (m == 0 || m == 32 || m == 64 || m == 128);
}

int scan_row_tiles(int G) { return G <= 4 ? 1 : (G <= 8 ? 2 : 4); }
bool scan_prepares_queries(const tq_codebook* ck, int G) { return scan_fused(scan_row_tiles(G), ck->spec.m); }

hipError_t launch_scan(const tq_codebook* ck, const tq_packed& k, const AttnArgs& a, const QDigits* q, int k0,
                       int klen, float* out, int64_t ld, int col0, hipStream_t stream) {
    const int G = a.Hq / a.h_kv;
    const int nrt = scan_row_tiles(G);
    const bool fused = scan_fused(nrt, ck->spec.m);
    if (fused != (q == nullptr)) return hipErrorInvalidValue;
    const int ngroups = (G + 4 * nrt - 1) / (4 * nrt);
    const bool paged = a.pages.table != nullptr;
    const int d = ck->spec.d, bits = ck->spec.bits, m = ck->spec.m;
    ScanFn fn = nullptr;
    if (d == 64) fn = paged ? pick_bits<64, true>(bits, nrt, m) : pick_bits<64, false>(bits, nrt, m);
    else if (d == 128) fn = paged ? pick_bits<128, true>(bits, nrt, m) : pick_bits<128, false>(bits, nrt, m);
    if (!fn) return hipErrorInvalidValue;
    ScanArgs p{};
    p.prep.q = a.q;
    p.prep.bf16 = a.bf16;
    p.prep.L_cap = a.L_cap;
    p.prep.norot = no_rotation(ck) ? 1 : 0;
    p.prep.s_ident = sign_corr(ck) ? 1 : 0;
    p.prep.rope_cos = a.rope_cos;
    p.prep.rope_sin = a.rope_sin;
    p.prep.sigma = ck->dev.sigma;
    p.prep.sketch_t = ck->dev.sketch_t;
    p.q_pos = a.q_pos;
    if (q) {
        p.qd = q->qd;
        p.sd = q->sd;
        p.scale = q->scale;
        p.sdw = q->sdw;
    }
    p.seq_len = a.seq_len;
    p.norm = k.norm;
    p.rnorm = k.rnorm;
    p.codes = k.codes;
    p.signs = k.signs;
    p.cap = paged ? a.pages.n_pages * a.h_kv * (int64_t)a.pages.size : (int64_t)a.B * a.h_kv * a.L_cap;
    p.Hq = a.Hq;
    p.h_kv = a.h_kv;
    p.L_cap = a.L_cap;
    p.m = m;
    p.ngroups = ngroups;
    p.k0 = k0;
    p.klen = klen;
    p.out = out;
    p.ld = ld;
    p.col0 = col0;
    for (int i = 0; i < 16; ++i) p.tdig[i] = ck->lvl_digits[i];
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
    // work per wave sized so that the whole grid is resident at once
    const int64_t gx = (int64_t)a.B * a.h_kv * ngroups;
    const int64_t tiles_row = (klen + 15) / 16;
    if (gx == 0 || tiles_row == 0) return hipSuccess;
    const int nwv = fused ? kFusedWaves : 4;
    const int64_t resident = resident_blocks((const void*)fn, 64 * nwv);
    const int64_t gy_want = std::max<int64_t>(1, (kScanRounds * resident + gx - 1) / gx);
    // a multiple of the prefetch depth per wave (the loop's step)
    const int pf = scan_depth(nrt, bits, paged);
    p.tiles_per_wave = (int)(((tiles_row + nwv * gy_want - 1) / (nwv * gy_want) + pf - 1) / pf * pf);
    const int64_t gy = (tiles_row + nwv * (int64_t)p.tiles_per_wave - 1) / (nwv * (int64_t)p.tiles_per_wave);
    hipLaunchKernelGGL(fn, dim3((unsigned)gx, (unsigned)gy), dim3(64 * nwv), 0, stream, p);
    return hipGetLastError();
}

}  // namespace tq
