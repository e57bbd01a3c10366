// Device-side building blocks shared by the logit scan (tq_logits.hip) and
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

// digit b of the levels of the 4 codes in the bytes of sel
__device__ __forceinline__ uint32_t lut4(const uint32_t* tdig, int b, uint32_t sel) {
    return __builtin_amdgcn_perm(tdig[2 * b + 1], tdig[2 * b], sel);
}

// v_perm selector for the 4 codes in the low 4*BITS bits of w: byte k = code k
template <int BITS>
__device__ __forceinline__ uint32_t code_sel(uint32_t w) {
    if constexpr (BITS == 3) {
        // even codes (bits 0-2, 6-8) and odd codes (3-5, 9-11) spread by
        // multiplication; the partial products never overlap
        return (((w & 0x1C7u) * 0x401u) & 0x70007u) | (((w & 0xE38u) * 0x8020u) & 0x7000700u);
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
__device__ __forceinline__ double digits4_value(const intx4& a) {
    const double h = (double)(a[0] * 128 + a[1]);  // |a| <= 2^25 per row: exact in int32
    const double l = (double)(a[2] * 128 + a[3]);
    return h * 16384.0 + l;
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
    // logit / nu = V qscale + gamma (Z zk - zc), Z the sign-digit sum
    double qscale[NRT], zk[NRT], zc[NRT];
    uint32_t tdig[8];

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
        const double tscale = ldexp(1.0, -lvl_shift);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const int g = gq0 + 4 * rt + qk;
            const int64_t row = rowbase + (g < G ? g : 0);
            qscale[rt] = ldexp(tscale, -(int)scale[row * 3 + 0]);
            // cq <s, z> with z = 2 bit - 1: (2 Z 2^-shift(s) - sum s) cq
            const double c = NCS > 0 ? cq : 0.0;
            zk[rt] = 2.0 * c * ldexp(1.0, -(int)scale[row * 3 + 1]);
            zc[rt] = c * (double)scale[row * 3 + 2];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) tdig[i] = lvl_digits[i];
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
                for (int bb = 0; bb < 3; ++bb) bd[c][bb][sg] = (int)lut4(tdig, bb, sel);
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
    // for the QJL sketch, the KV head's mu for the sign correction
    __device__ void finish(const Acc& A, float gm, double out[NRT]) const {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            // y[b][a]: digit a of q' (weight 2^(7(3-a))) times digit b of t
            // (weight 2^(8(2-b))); |y| <= 128 * 64 * 128 = 2^20
            double V = 0.0;
#pragma unroll
            for (int bb = 0; bb < 3; ++bb) V = V * 256.0 + digits4_value(A.y[rt][bb]);
            double logit = V * qscale[rt];
            if constexpr (NCS > 0) {
                // sum_l s_l z_l = 2 sum_l s_l bit_l - sum_l s_l; the digit rows
                // are paired in int32 (|z| <= 64 * 64 per row)
                const intx4& z = A.z[rt];
                const double Z = digits4_value(z);
                logit = fma((double)gm, fma(Z, zk[rt], -zc[rt]), logit);
            }
            out[rt] = logit;
        }
    }

    __device__ void compute(const Raw& r, float gm, int per, int lane, double out[NRT]) const {
        Acc A;
        mma(r, per, lane, A);
        finish(A, gm, out);
    }
};

}  // namespace dev
}  // namespace tq
