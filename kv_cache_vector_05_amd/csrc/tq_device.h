// Device-side building blocks shared by the logit scan (tq_scan.hip) and
// the fused decode (tq_decode.hip): code unpacking into v_perm selectors,
// level-digit lookup, sign-bit spreading, and the integer-MFMA logit of one
// 16-key tile.
//
// Logit of one key (iaemfoco post, "TurboQuant: Uma Nova Abordagem"; itstec
// post, "Por dentro do processo de compressao KV"):
//     logit = nu ( <q', t[c]> + sqrt(pi/2)/m * gamma * <s, z> ),  q' = Pi RoPE(q), s = S q'.
// Every operand is an exact fixed-point integer split into int8 digits (q'
// and s: 28 bits in four balanced base-128 digits; levels: 24 bits in three
// balanced base-256 digits); v_mfma_i32_16x16x64_i8 sums the digit products
// exactly and only the combination of the digit sums is rounded.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tq {
namespace dev {

typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx2 __attribute__((ext_vector_type(2)));

constexpr double kQjlD = 1.2533141373155003;  // sqrt(pi / 2)

__device__ __forceinline__ int clamp_len(const int32_t* seq_len, int b, int L_cap) {
    int s = seq_len[b];
    return s < 0 ? 0 : (s > L_cap ? L_cap : s);
}

// RoPE position of sequence b's query: q_pos[b] when a position array is
// given, else seq_len[b] (the token after the cached ones); clamped to [0, L_cap]
__device__ __forceinline__ int query_pos(const int32_t* q_pos, const int32_t* seq_len, int b, int L_cap) {
    int s = q_pos ? q_pos[b] : seq_len[b];
    return s < 0 ? 0 : (s > L_cap ? L_cap : s);
}

// Division by a run-time constant d >= 1 for dividends below 2^31, by a
// multiply-high and a shift (Granlund and Montgomery, PLDI 1994): with
// s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d) + 1,
// n / d = (mulhi(n, m) + n) >> s.  Set up on the host.
struct FastDiv {
    uint32_t d, m, s;
    __host__ __device__ FastDiv() : d(1), m(0), s(0) {}
    __host__ explicit FastDiv(uint32_t div) : d(div) {
        s = 0;
        while ((1ull << s) < div) ++s;
        m = (uint32_t)(((1ull << 32) * ((1ull << s) - div)) / div + 1);
    }
    __device__ uint32_t div(uint32_t n) const { return (__umulhi(n, m) + n) >> s; }
};

// digit b of the levels of the 4 codes in the bytes of sel.  tdig holds the
// digits of levels 0-7 in words 2b, 2b + 1 and of levels 8-15 in words
// 8 + 2b, 8 + 2b + 1 (byte c % 4 of word c / 4 of its half).  Up to 8
// levels: one v_perm; 16 levels: one per half and a byte select on bit 3 of
// each code (v_perm selectors 8-15 would not index bytes).
template <int BITS>
__device__ __forceinline__ uint32_t lut(const uint32_t* tdig, int b, uint32_t sel) {
    if constexpr (BITS <= 3) {
        return __builtin_amdgcn_perm(tdig[2 * b + 1], tdig[2 * b], sel);
    } else {
        const uint32_t s7 = sel & 0x07070707u;
        const uint32_t lo = __builtin_amdgcn_perm(tdig[2 * b + 1], tdig[2 * b], s7);
        const uint32_t hi = __builtin_amdgcn_perm(tdig[8 + 2 * b + 1], tdig[8 + 2 * b], s7);
        const uint32_t mask = ((sel >> 3) & 0x01010101u) * 0xFFu;
        return (hi & mask) | (lo & ~mask);
    }
}

// v_perm selector for the 4 codes in the low 4*BITS bits of w: byte k = code k
template <int BITS>
__device__ __forceinline__ uint32_t code_sel(uint32_t w) {
    if constexpr (BITS == 3) {
        // even codes (bits 0-2, 6-8) and odd codes (3-5, 9-11) spread by
        // multiplication; the partial products never overlap
        return (((w & 0x1C7u) * 0x401u) & 0x70007u) | (((w & 0xE38u) * 0x8020u) & 0x7000700u);
    } else if constexpr (BITS == 4) {
        // nibbles 0, 1 to bytes 0, 1 and nibbles 2, 3 to bytes 2, 3
        const uint32_t t = __builtin_amdgcn_perm(0u, w, 0x0C010C00u);  // bytes: w0, 0, w1, 0
        return (t & 0x000F000Fu) | ((t & 0x00F000F0u) << 4);
    } else if constexpr (BITS == 2) {
        return (((w & 0x33u) * 0x1001u) & 0x30003u) | (((w & 0xCCu) * 0x40040u) & 0x3000300u);
    } else {
        return ((w & 0xFu) * 0x204081u) & 0x01010101u;
    }
}

// Where coordinate i's code sits in a record's code words: its low n0 bits
// at word w0 from bit s0, the rest (if n0 < bits) at word w1 from bit s1.
//  * 1, 2 and 4 bits: bits [b*i, b*i+b) of the LSB-first bit string.
//  * 3 bits: groups of 32 coordinates in three words W0..W2.  Coordinate
//    j < 24 of a group takes bits 8(j%4) + 3((j%8)/4) .. +2 of W_{j/8} (two
//    whole codes per byte); for j = 24 + r the low two bits sit at bit
//    8(r%4) + 6 of W_{r/4} and the high bit at bit 8(r%4) + 6 + r/4 of W2.
//    A byte-wise mask then yields four codes at once (see Quarter::sel).
struct CodeLoc {
    int w0, s0, n0, w1, s1;
};
__host__ __device__ constexpr CodeLoc code_loc(int i, int bits) {
    if (bits == 3) {
        const int g = i >> 5, j = i & 31;
        if (j < 24) return CodeLoc{3 * g + (j >> 3), 8 * (j & 3) + 3 * ((j & 7) >> 2), 3, 0, 0};
        const int r = j - 24;
        return CodeLoc{3 * g + (r >> 2), 8 * (r & 3) + 6, 2, 3 * g + 2, 8 * (r & 3) + 6 + (r >> 2)};
    }
    const int bp = bits * i, s0 = bp & 31;
    return CodeLoc{bp >> 5, s0, (32 - s0) < bits ? (32 - s0) : bits, (bp >> 5) + 1, 0};
}
__host__ __device__ inline uint32_t code_get(const uint32_t* cw, const CodeLoc& L, int bits) {
    uint32_t c = (cw[L.w0] >> L.s0) & ((1u << L.n0) - 1u);
    if (L.n0 < bits) c |= ((cw[L.w1] >> L.s1) & ((1u << (bits - L.n0)) - 1u)) << L.n0;
    return c;
}
// ORs code c (< 2^bits) into zero-initialised words
__host__ __device__ inline void code_put(uint32_t* cw, const CodeLoc& L, int bits, uint32_t c) {
    cw[L.w0] |= (L.n0 == bits ? c : (c & ((1u << L.n0) - 1u))) << L.s0;
    if (L.n0 < bits) cw[L.w1] |= (c >> L.n0) << L.s1;
}

// bytes 0..3 of the result = bits 0..3 of x (as 0/1)
__device__ __forceinline__ uint32_t spread4(uint32_t x) { return ((x & 0xFu) * 0x204081u) & 0x01010101u; }

// bytes 0..3 of the result = bits 0..3 of x as +1 (bit set) / -1 (bit clear)
__device__ __forceinline__ uint32_t spread4_pm(uint32_t x) { return 0xFFFFFFFFu ^ (spread4(x) * 0xFEu); }

// Code bits of one lane's coordinate quarter [qk*D/4, (qk+1)*D/4) of a
// record, and the v_perm selectors (byte u = code of coordinate 4g + u of
// the quarter) built from them.
template <int D, int BITS>
struct Quarter {
    static constexpr int LPG = D / 4;         // coordinates per quarter
    static constexpr int CW = BITS * D / 32;  // code words per record
    static constexpr int BPG = BITS * LPG;    // code bits per quarter
    static constexpr bool ALIGNED = (BPG % 32) == 0;
    // 3 bits: the whole 32-coordinate group holding the quarter
    static constexpr int NW = BITS == 3 ? 3 : (ALIGNED ? BPG / 32 : (BPG + 31) / 32 + 1);

    // offset (words) of the first word the lane loads
    __device__ static int word0(int qk) {
        if constexpr (BITS == 3) return 3 * ((LPG * qk) >> 5);
        return (BPG * qk) >> 5;
    }

    // cp points at word word0(qk) of the record
    __device__ static void load(const uint32_t* cp, int qk, uint32_t W[NW]) {
        if constexpr (BITS == 3 || ALIGNED) {
#pragma unroll
            for (int i = 0; i < NW; ++i) W[i] = cp[i];
        } else {
            const int w0 = word0(qk);
#pragma unroll
            for (int i = 0; i < NW; ++i) W[i] = cp[min(i, CW - 1 - w0)];
            const int sh = (BPG * qk) & 31;
#pragma unroll
            for (int i = 0; i + 1 < NW; ++i) W[i] = __builtin_amdgcn_alignbit(W[i + 1], W[i], sh);
        }
    }

    // selector t (0..7) of a 3-bit group: codes of coordinates 4t .. 4t+3
    __device__ static uint32_t group_sel(const uint32_t W[3], int t) {
        constexpr uint32_t M3 = 0x07070707u, M2 = 0x03030303u, M1 = 0x04040404u;
        switch (t) {
            case 0: return W[0] & M3;
            case 1: return (W[0] >> 3) & M3;
            case 2: return W[1] & M3;
            case 3: return (W[1] >> 3) & M3;
            case 4: return W[2] & M3;
            case 5: return (W[2] >> 3) & M3;
            case 6: return ((W[0] >> 6) & M2) | ((W[2] >> 4) & M1);
            default: return ((W[1] >> 6) & M2) | ((W[2] >> 5) & M1);
        }
    }

    // v_perm selector of coordinates 4g .. 4g+3 of the quarter
    __device__ static uint32_t sel(const uint32_t W[NW], int g, int qk) {
        if constexpr (BITS == 3) {
            if constexpr (LPG == 32) return group_sel(W, g);
            // half a group: quarters with odd qk hold coordinates 16..31
            const uint32_t lo = group_sel(W, g), hi = group_sel(W, 4 + g);
            return (qk & 1) ? hi : lo;
        } else {
            const int o = BITS * 4 * g;
            const uint32_t lo = W[o >> 5];
            const uint32_t hi = ((o >> 5) + 1 < NW) ? W[(o >> 5) + 1] : 0u;
            return code_sel<BITS>(__builtin_amdgcn_alignbit(hi, lo, o & 31));
        }
    }
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// buffer resource over [base, base + bytes) (gfx9 word 3: 32-bit elements, no
// swizzle); loads past the end return 0
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int64_t bytes) {
    const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

// Quarter<D, BITS>::load through a buffer resource: voff is the byte offset of
// the lane's record word word0(qk), soff a scalar byte offset; no vector
// address arithmetic
template <int D, int BITS>
__device__ __forceinline__ void quarter_load_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, int qk,
                                                 uint32_t* W) {
    using Q = Quarter<D, BITS>;
    if constexpr (Q::NW == 3) {
        const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, 0);
        W[0] = v.x;
        W[1] = v.y;
        W[2] = v.z;
    } else if constexpr (Q::NW == 4 && Q::ALIGNED) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
        W[0] = v.x;
        W[1] = v.y;
        W[2] = v.z;
        W[3] = v.w;
    } else if constexpr (Q::NW == 2 && Q::ALIGNED) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
        W[0] = v.x;
        W[1] = v.y;
    } else if constexpr (Q::ALIGNED) {
#pragma unroll
        for (int i = 0; i < Q::NW; ++i) W[i] = __builtin_amdgcn_raw_buffer_load_b32(r, voff + 4u * i, soff, 0);
    } else {
        // the quarter straddles words: NW words from word0, the last clamped
        // into the record, shifted into place
        const int w0 = Q::word0(qk);
#pragma unroll
        for (int i = 0; i < Q::NW; ++i)
            W[i] = __builtin_amdgcn_raw_buffer_load_b32(r, voff + 4u * (uint32_t)min(i, Q::CW - 1 - w0), soff, 0);
        const int sh = (Q::BPG * qk) & 31;
#pragma unroll
        for (int i = 0; i + 1 < Q::NW; ++i) W[i] = __builtin_amdgcn_alignbit(W[i + 1], W[i], sh);
    }
}

// Fixed point with four balanced base-128 digits: x ~= X * 2^-sh, |X| <= 2^26.
__device__ __forceinline__ int fixed_shift(float amax) {
    if (!(amax > 0.0f)) return 0;
    int e;
    frexpf(amax, &e);
    return 26 - e;
}

// four balanced base-128 digits of |X| < 2^27 packed in bytes (byte a = digit a,
// most significant first): X = sum_a d_a 128^(3-a)
__device__ __forceinline__ uint32_t digits4_packed(int X) {
    const int r3 = ((X + 64) & 127) - 64;
    X = (X - r3) >> 7;
    const int r2 = ((X + 64) & 127) - 64;
    X = (X - r2) >> 7;
    const int r1 = ((X + 64) & 127) - 64;
    const int r0 = (X - r1) >> 7;
    return (uint32_t)(r0 & 0xFF) | ((uint32_t)(r1 & 0xFF) << 8) | ((uint32_t)(r2 & 0xFF) << 16) |
           ((uint32_t)(r3 & 0xFF) << 24);
}

// value of an MFMA result whose four rows are the base-128 digits of one operand
// value of four digit rows (base 128, most significant first) as a float:
// the row pairs combine exactly in int32 (|a| <= 2^20 per row), and the pair
// sum rounds once
__device__ __forceinline__ float digits4_f32(const intx4& a) {
    return fmaf((float)(a[0] * 128 + a[1]), 16384.0f, (float)(a[2] * 128 + a[3]));
}

// Exact logit of one 16-key tile on the int8 matrix cores.
//
// MFMA shape: rows = (query, digit of q') - four digits of four queries fill
// the 16 rows - columns = 16 keys, K = 64 coordinates.  Lane l owns key l % 16
// and the coordinate quarter qk = l / 16; its 16 K-slots per MFMA are 16
// consecutive coordinates.  The B operand (digit b of t[c] for those
// coordinates) is built with one v_perm per 4 coordinates from an 8-byte
// digit table.  After the MFMAs lane l holds the logit of (query 4 rt + l/16,
// key l % 16) of each row tile rt.
template <int D, int BITS, int NRT, int NCS>
struct TileLogit {
    using Q = Quarter<D, BITS>;
    static constexpr int NC = Q::LPG / 16;  // K=64 chunks over the coordinates

    intx4 aq[NRT][NC];
    intx4 as[NRT][NCS > 0 ? NCS : 1];
    // logit / nu = V 2^qe + gamma (Z 2^ze c2 - zc), Z the sign-digit sum (the
    // powers of two are applied by ldexp, so no scale leaves the fp32 range)
    int qe[NRT], ze[NRT];
    float c2[NRT], zc[NRT];
    uint32_t tdig[16];

    // qd/sd/scale: the prepared query digits; cq: scale of the correction
    // term (sqrt(pi/2)/m for the QJL sketch, 1 for the sign correction);
    // rowbase: first query row of the KV head; gq0: first query of this
    // row-tile set; G: queries per KV head
    __device__ void init(const int8_t* qd, const int8_t* sd, const float* scale, int sdw, double cq, int64_t rowbase,
                         int gq0, int G, const uint32_t* lvl_digits, int lvl_shift, int lane) {
        const int qk = lane >> 4;
        const int a = lane & 3;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const int g = gq0 + 4 * rt + ((lane & 15) >> 2);
            const bool ok = g < G;
            const int64_t drow = (rowbase + (ok ? g : 0)) * 4 + a;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const intx4 v = *reinterpret_cast<const intx4*>(qd + drow * D + qk * Q::LPG + 16 * c);
                aq[rt][c] = ok ? v : intx4{0, 0, 0, 0};
            }
#pragma unroll
            for (int cs = 0; cs < NCS; ++cs) {
                const intx4 v = *reinterpret_cast<const intx4*>(sd + drow * sdw + (qk * NCS + cs) * 16);
                as[rt][cs] = ok ? v : intx4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const int g = gq0 + 4 * rt + qk;
            const int64_t row = rowbase + (g < G ? g : 0);
            qe[rt] = -lvl_shift - (int)scale[row * 3 + 0];
            // cq <s, z> with z = 2 bit - 1: (2 Z 2^-shift(s) - sum s) cq
            const double c = NCS > 0 ? cq : 0.0;
            ze[rt] = -(int)scale[row * 3 + 1];
            c2[rt] = (float)(2.0 * c);
            zc[rt] = (float)(c * (double)scale[row * 3 + 2]);
        }
#pragma unroll
        for (int i = 0; i < (BITS == 4 ? 16 : 8); ++i) tdig[i] = lvl_digits[i];
    }

    // The lane's share of one key record, loaded ahead of its use so that a
    // tile's loads can be in flight while the previous tile computes.
    struct Raw {
        uint32_t W[Q::NW];
        uint32_t sg;  // the sign word holding the lane's sketch rows (m <= 128)
    };

    // cp: word Q::word0(qk) of the key's code words; sp: the key's sign words;
    // per = m / 4 sketch rows per lane group
    __device__ static void load(const uint32_t* cp, const uint32_t* sp, int per, int lane, Raw& r) {
        const int qk = lane >> 4;
        Q::load(cp, qk, r.W);
        r.sg = NCS > 0 ? sp[(qk * per) >> 5] : 0u;
    }

    // integer digit sums of one tile (before their combination)
    struct Acc {
        intx4 y[NRT][3];
        intx4 z[NRT];
    };

    __device__ void mma(const Raw& r, int per, int lane, Acc& A) const {
        const int qk = lane >> 4;
        intx4 bd[NC][3];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int sg = 0; sg < 4; ++sg) {
                const uint32_t sel = Q::sel(r.W, 4 * c + sg, qk);
#pragma unroll
                for (int bb = 0; bb < 3; ++bb) bd[c][bb][sg] = (int)lut<BITS>(tdig, bb, sel);
            }
        }
        intx4 bz[NCS > 0 ? NCS : 1];
        if constexpr (NCS > 0) {
#pragma unroll
            for (int cs = 0; cs < NCS; ++cs) {
                const int bit0 = qk * per + 16 * cs;  // within the word loaded into r.sg
                uint32_t x = r.sg >> (bit0 & 31);
                if (per - 16 * cs < 16) x &= (1u << (per - 16 * cs)) - 1u;  // fewer than 16 rows left
                bz[cs][0] = (int)spread4(x);
                bz[cs][1] = (int)spread4(x >> 4);
                bz[cs][2] = (int)spread4(x >> 8);
                bz[cs][3] = (int)spread4(x >> 12);
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
    }

    // out[rt] = <q', t[c]> + cq gm <s, z>  (not yet times nu); gm is gamma
    // for the QJL sketch, the KV head's mu for the sign correction.  The digit
    // sums are exact; their combination runs in fp32, whose roundings stay
    // near 2^-22 of max(|logit|, 2^-7 sum_i |q'_i t_i|) (the top digits carry
    // the sum to within that fraction), far inside the logits' tolerance.
    __device__ void finish(const Acc& A, float gm, float out[NRT]) const {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            // y[b][a]: digit a of q' (weight 2^(7(3-a))) times digit b of t
            // (weight 2^(8(2-b))); |y| <= 128 * 64 * 128 = 2^20
            float V = 0.0f;
#pragma unroll
            for (int bb = 0; bb < 3; ++bb) V = fmaf(V, 256.0f, digits4_f32(A.y[rt][bb]));
            float logit = ldexpf(V, qe[rt]);
            if constexpr (NCS > 0) {
                // sum_l s_l z_l = 2 sum_l s_l bit_l - sum_l s_l; the digit rows
                // are paired in int32 (|z| <= 64 * 64 per row)
                const float Z = ldexpf(digits4_f32(A.z[rt]), ze[rt]);
                logit = fmaf(gm, fmaf(Z, c2[rt], -zc[rt]), logit);
            }
            out[rt] = logit;
        }
    }

    __device__ void compute(const Raw& r, float gm, int per, int lane, float out[NRT]) const {
        Acc A;
        mma(r, per, lane, A);
        finish(A, gm, out);
    }
};

// ---------------------------------------------------------------- query preparation
// q' = Pi RoPE(q) and s = S q' (s = q' with the sign correction of the
// TurboESM summary, technical section 2), as fixed-point integers with one
// power-of-two scale per query (|X| <= 2^26) split into four balanced
// base-128 int8 digits: the A operands of the integer-MFMA logit tile (tambur
// post: logits straight from quantised keys; iaemfoco post, "TurboQuant: Uma
// Nova Abordagem": the QJL correction), with the scale and the exact sum of
// the fixed-point s values beside them.

__device__ __forceinline__ long long to_fixed(float x, int sh) { return llrint(ldexp((double)x, sh)); }
// four balanced base-128 digits of X (most significant first)
__device__ __forceinline__ void digits4(long long X, int8_t d[4]) {
#pragma unroll
    for (int k = 3; k >= 1; --k) {
        long long r = ((X + 64) & 127) - 64;
        d[k] = (int8_t)r;
        X = (X - r) >> 7;
    }
    d[0] = (int8_t)X;
}
__device__ __forceinline__ float wave_max64(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ double wave_sum64(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

struct PrepIn {
    const void* q;            // [rows][d] float32 or bfloat16
    int32_t bf16, L_cap;
    int32_t norot;            // Pi = I: q' = RoPE(q)
    int32_t s_ident;          // S = I (sign correction): s = q'
    const float* rope_cos;    // [n_pos][d/2] or nullptr
    const float* rope_sin;
    const float* sigma;       // Hadamard signs
    const float* sketch_t;    // S^T [d][m]
};

// LDS of the preparation of R query rows (ST threads sum the sketch)
template <int D, int M, int R, int ST = 256>
struct alignas(16) PrepLds {
    static constexpr int NCS = M == 0 ? 0 : (M >= 64 ? M / 64 : 1);  // 64-row sketch chunks of the MFMA
    static constexpr int SDW = 64 * (NCS > 0 ? NCS : 1);             // bytes per digit row of s
    float qp[R][D];               // q'
    float part[M > 0 ? R : 1][ST];  // partial sums of s (one per thread)
    float s[R][M > 0 ? M : 1];
    int8_t qd[R][4][D];           // digit rows of q'
    int8_t sd[R][4][SDW];         // digit rows of s in MFMA slot order
    float scl[R][3];              // shift(q'), shift(s), sum of the fixed-point s values
};

// Preparation of R query rows by the first four waves of a workgroup (the
// sketch product by its first ST threads), in two stages so that a caller can put other loads in flight behind the
// preparation's own: load() issues every load, compute() waits for them and
// fills the LDS (ending with a barrier).  Every load is unconditional, through
// a buffer resource (one of size zero reads zeros where an input is absent),
// and the query rows go first: with no load behind a branch the in-order
// count of outstanding loads stays exact, so compute() waits for the operand
// it needs next and the loads issued after it (the sketch, the caller's
// record prefetch) stay in flight.  Row r is query row
// row_of(min(r, R - 1)); waves 0-3 prepare rows w, w + 4, ...  Thread
// (part, l) of the first ST sums row l of S over one of ST/m coordinate
// ranges, so each entry of S is read once and a wave's loads are
// contiguous; a wider workgroup's other waves only pass the barriers (their
// sketch loads fall past S and read nothing).
template <int D, int M, int R, int ST = 256>
struct Prep {
    static_assert(ST >= 256 && ST % 256 == 0, "the sketch takes whole groups of four waves");
    static constexpr int VPL = D / 64;
    static constexpr int NT = M > 0 ? ST / M : 1;  // parts per sketch row
    static constexpr int NI = D / NT;               // S^T entries per thread
    static constexpr int RW = (R + 3) / 4;          // rows per wave
    // raw words as loaded; compute() converts them
    uint32_t sk[M > 0 ? NI : 1];
    uint32_t xw[RW][VPL];  // fp32, or the aligned word holding the bf16 element
    uint32_t sgw[VPL];
    uint32_t cw = 0u, snw = 0u;

    // pos: the queries' RoPE position (one sequence per workgroup)
    template <typename RowOf>
    __device__ void load(const PrepIn& in, RowOf row_of, int pos) {
        const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
        // query element e: word e (fp32) or the word holding bf16 element e
        // (the other half is its neighbour; rows have an even length)
        const __amdgpu_buffer_rsrc_t rq = buf_rsrc(in.q, 0xFFFFFFFFll);
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            const int64_t row = row_of(min(wave + 4 * j, R - 1));
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                const uint32_t e = (uint32_t)(row * D + lane + 64 * v);
                xw[j][v] = __builtin_amdgcn_raw_buffer_load_b32(rq, in.bf16 ? (2u * e) & ~3u : 4u * e, 0, 0);
            }
        }
        const __amdgpu_buffer_rsrc_t rsg = buf_rsrc(in.sigma, in.norot ? 0 : D * 4);
#pragma unroll
        for (int v = 0; v < VPL; ++v) sgw[v] = __builtin_amdgcn_raw_buffer_load_b32(rsg, 4u * (lane + 64 * v), 0, 0);
        const int64_t rope_bytes = in.rope_cos ? ((int64_t)in.L_cap + 1) * (D / 2) * 4 : 0;
        const __amdgpu_buffer_rsrc_t rc = buf_rsrc(in.rope_cos, rope_bytes), rsn = buf_rsrc(in.rope_sin, rope_bytes);
        const uint32_t ro = 4u * (uint32_t)(pos * (D / 2) + lane % (D / 2));
        cw = __builtin_amdgcn_raw_buffer_load_b32(rc, ro, 0, 0);
        snw = __builtin_amdgcn_raw_buffer_load_b32(rsn, ro, 0, 0);
        if constexpr (M > 0) {
            const __amdgpu_buffer_rsrc_t rsk = buf_rsrc(in.sketch_t, in.s_ident ? 0 : D * M * 4);
            const int l = t % M, prt = t / M;
#pragma unroll
            for (int k = 0; k < NI; ++k)
                sk[k] = __builtin_amdgcn_raw_buffer_load_b32(rsk, 4u * (uint32_t)((prt * NI + k) * M + l), 0, 0);
        }
    }

    __device__ void compute(const PrepIn& in, PrepLds<D, M, R, ST>& L) {
        const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            const int r = wave + 4 * j;
            if (r >= R || wave >= 4) break;  // the same for the whole wave
            float xv[VPL];
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                const uint32_t w = xw[j][v];
                xv[v] = __uint_as_float(in.bf16 ? ((lane & 1) ? w & 0xFFFF0000u : w << 16) : w);
            }
            const float c = __uint_as_float(cw), sn = __uint_as_float(snw);
            if (in.rope_cos) {
                // RoPE: pair (i, i + d/2) in one lane (d = 128) or lanes l, l ^ 32 (d = 64)
                if constexpr (VPL == 2) {
                    const float lo = xv[0], hi = xv[1];
                    xv[0] = lo * c - hi * sn;
                    xv[1] = hi * c + lo * sn;
                } else {
                    const float own = xv[0], other = __shfl_xor(own, 32);
                    xv[0] = lane < 32 ? own * c - other * sn : own * c + other * sn;
                }
            }
            if (!in.norot) {
#pragma unroll
                for (int v = 0; v < VPL; ++v) xv[v] *= __uint_as_float(sgw[v]);
                // H_d in Sylvester order: butterflies over every index bit
#pragma unroll
                for (int sp = 1; sp < 64; sp <<= 1) {
#pragma unroll
                    for (int v = 0; v < VPL; ++v) {
                        const float o = __shfl_xor(xv[v], sp);
                        xv[v] = (lane & sp) ? o - xv[v] : xv[v] + o;
                    }
                }
                if constexpr (VPL == 2) {
                    const float a0 = xv[0], a1 = xv[1];
                    xv[0] = a0 + a1;
                    xv[1] = a0 - a1;
                }
                const float inv = 1.0f / sqrtf((float)D);
#pragma unroll
                for (int v = 0; v < VPL; ++v) xv[v] *= inv;
            }
            float amax = 0.0f;
#pragma unroll
            for (int v = 0; v < VPL; ++v) amax = fmaxf(amax, fabsf(xv[v]));
            const int shq = fixed_shift(wave_max64(amax));
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                const int i = lane + 64 * v;
                L.qp[r][i] = xv[v];
                int8_t d[4];
                digits4(to_fixed(xv[v], shq), d);
#pragma unroll
                for (int a = 0; a < 4; ++a) L.qd[r][a][i] = d[a];
            }
            if (lane == 0) {
                L.scl[r][0] = (float)shq;  // shifts are small integers, exact in fp32
                L.scl[r][1] = 0.0f;
                L.scl[r][2] = 0.0f;
            }
        }
        if constexpr (M > 0) {
            const bool sketch = !in.s_ident;
            __syncthreads();
            // partial sums of s = S q' (or s = q')
            if (sketch && t < ST) {
                const int prt = t / M;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float acc = 0.0f;
#pragma unroll
                    for (int k = 0; k < NI; ++k) acc = fmaf(__uint_as_float(sk[k]), L.qp[r][prt * NI + k], acc);
                    L.part[r][t] = acc;
                }
            }
            __syncthreads();
            for (int idx = t; t < 256 && idx < R * M; idx += 256) {
                const int r = idx / M, l = idx % M;
                float sv = 0.0f;
                if (sketch) {
#pragma unroll
                    for (int k = 0; k < NT; ++k) sv += L.part[r][k * M + l];
                } else {
                    sv = L.qp[r][l];
                }
                L.s[r][l] = sv;
            }
            __syncthreads();
            // scale, exact sum and digits of s; digit byte (qk*ncs + cs)*16 + j
            // holds sketch row qk*(m/4) + 16*cs + j (zero where that slot is past m/4)
            constexpr int NCS = PrepLds<D, M, R, ST>::NCS, SDW = PrepLds<D, M, R, ST>::SDW;
#pragma unroll
            for (int j = 0; j < RW; ++j) {
                const int r = wave + 4 * j;
                if (r >= R || wave >= 4) break;
                float smax = 0.0f;
                double sf = 0.0;
                for (int li = lane; li < M; li += 64) smax = fmaxf(smax, fabsf(L.s[r][li]));
                const int shs = fixed_shift(wave_max64(smax));
                for (int li = lane; li < M; li += 64) sf += (double)to_fixed(L.s[r][li], shs);
                sf = wave_sum64(sf);
                for (int off = lane; off < SDW; off += 64) {
                    const int qk = off / (16 * NCS), rem = off % (16 * NCS);
                    const int cs = rem / 16, jj = rem % 16;
                    int8_t d[4] = {0, 0, 0, 0};
                    if (16 * cs + jj < M / 4) digits4(to_fixed(L.s[r][qk * (M / 4) + 16 * cs + jj], shs), d);
#pragma unroll
                    for (int a = 0; a < 4; ++a) L.sd[r][a][off] = d[a];
                }
                if (lane == 0) {
                    L.scl[r][1] = (float)shs;
                    L.scl[r][2] = (float)ldexp(sf, -shs);
                }
            }
        }
        __syncthreads();
    }
};

}  // namespace dev
}  // namespace tq
