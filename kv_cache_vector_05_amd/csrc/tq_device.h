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

// bytes 0..3 of the result = bits 0..3 of x (as 0/1)
__device__ __forceinline__ uint32_t spread4(uint32_t x) { return ((x & 0xFu) * 0x204081u) & 0x01010101u; }

// bytes 0..3 of the result = bits 0..3 of x as +1 (bit set) / -1 (bit clear)
__device__ __forceinline__ uint32_t spread4_pm(uint32_t x) { return 0xFFFFFFFFu ^ (spread4(x) * 0xFEu); }

// Code bits of one lane's coordinate quarter [qk*D/4, (qk+1)*D/4) of a
// record, shifted so that coordinate qk*D/4 starts at bit 0 of W[0].
template <int D, int BITS>
struct Quarter {
    static constexpr int LPG = D / 4;           // coordinates per quarter
    static constexpr int CW = BITS * D / 32;    // code words per record
    static constexpr int BPG = BITS * LPG;      // code bits per quarter
    static constexpr bool ALIGNED = (BPG % 32) == 0;
    static constexpr int NW = ALIGNED ? BPG / 32 : (BPG + 31) / 32 + 1;

    // offset (words) of the quarter's first word within a record
    __device__ static int word0(int qk) { return (BPG * qk) >> 5; }

    // cp points at word word0(qk) of the record
    __device__ static void load(const uint32_t* cp, int qk, uint32_t W[NW]) {
        if constexpr (ALIGNED) {
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

    // v_perm selector of coordinates 4*g .. 4*g+3 of the quarter
    __device__ static uint32_t sel(const uint32_t W[NW], int g) {
        const int o = BITS * 4 * g;
        const uint32_t lo = W[o >> 5];
        const uint32_t hi = ((o >> 5) + 1 < NW) ? W[(o >> 5) + 1] : 0u;
        return code_sel<BITS>(__builtin_amdgcn_alignbit(hi, lo, o & 31));
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
    double qscale[NRT], sscale[NRT], ssum[NRT];
    double cq;
    uint32_t tdig[8];

    // qd/sd/scale: the prepared query digits; rowbase: first query row of the
    // KV head; gq0: first query of this row-tile set; G: queries per KV head
    __device__ void init(const int8_t* qd, const int8_t* sd, const float* scale, int sdw, int m, int64_t rowbase,
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
            sscale[rt] = ldexp(1.0, -(int)scale[row * 3 + 1]);
            ssum[rt] = (double)scale[row * 3 + 2];
        }
        cq = NCS > 0 ? kQjlD / (double)m : 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) tdig[i] = lvl_digits[i];
    }

    // cp: the lane's code words (word Q::word0(qk) of its key's record);
    // sp: the key's sign words; per = m / 4 sketch rows per lane group;
    // out[rt] = <q', t[c]> + sqrt(pi/2)/m gamma <s, z>  (not yet times nu)
    __device__ void compute(const uint32_t* cp, const uint32_t* sp, float gm, int per, int lane, double out[NRT]) const {
        const int qk = lane >> 4;
        uint32_t W[Q::NW];
        Q::load(cp, qk, W);
        intx4 bd[NC][3];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int sg = 0; sg < 4; ++sg) {
                const uint32_t sel = Q::sel(W, 4 * c + sg);
#pragma unroll
                for (int bb = 0; bb < 3; ++bb) bd[c][bb][sg] = (int)lut4(tdig, bb, sel);
            }
        }
        intx4 bz[NCS > 0 ? NCS : 1];
        if constexpr (NCS > 0) {
#pragma unroll
            for (int cs = 0; cs < NCS; ++cs) {
                const int bit0 = qk * per + 16 * cs;
                uint32_t x = sp[bit0 >> 5] >> (bit0 & 31);
                if (per - 16 * cs < 16) x &= (1u << (per - 16 * cs)) - 1u;  // fewer than 16 rows left
                bz[cs][0] = (int)spread4(x);
                bz[cs][1] = (int)spread4(x >> 4);
                bz[cs][2] = (int)spread4(x >> 8);
                bz[cs][3] = (int)spread4(x >> 12);
            }
        }
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            intx4 acc[3];
#pragma unroll
            for (int bb = 0; bb < 3; ++bb) acc[bb] = intx4{0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int bb = 0; bb < 3; ++bb)
                    acc[bb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[rt][c], bd[c][bb], acc[bb], 0, 0, 0);
            intx4 accz = intx4{0, 0, 0, 0};
#pragma unroll
            for (int cs = 0; cs < NCS; ++cs)
                accz = __builtin_amdgcn_mfma_i32_16x16x64_i8(as[rt][cs], bz[cs], accz, 0, 0, 0);
            // acc[b][a]: digit a of q' (weight 2^(7(3-a))) times digit b of t
            // (weight 2^(8(2-b))); |acc| <= 128 * 64 * 128 = 2^20
            double V = 0.0;
#pragma unroll
            for (int bb = 0; bb < 3; ++bb) V = V * 256.0 + digits4_value(acc[bb]);
            double logit = V * qscale[rt];
            if constexpr (NCS > 0) {
                // sum_l s_l z_l = 2 sum_l s_l bit_l - sum_l s_l
                const double Z = ((double)accz[0] * 2097152.0 + (double)accz[1] * 16384.0) +
                                 ((double)accz[2] * 128.0 + (double)accz[3]);
                logit += cq * (double)gm * (2.0 * Z * sscale[rt] - ssum[rt]);
            }
            out[rt] = logit;
        }
    }
};

}  // namespace dev
}  // namespace tq
