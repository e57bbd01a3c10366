// Encoder kernels (FibQuant summary, sections 1 and 2.3; iaemfoco post,
// "TurboQuant: Uma Nova Abordagem"; itstec post, "Por dentro do processo de
// compressao KV"; TurboESM summary, technical section 2 for RoPE first).
//
// Hadamard form (d = 64 or 128): one wave64 encodes a tile of 32 consecutive
// tokens of one (sequence, head); lane l serves vector l % 32 with lane half
// h = l / 32.
//   * Input step kb holds coordinates 16 kb + 8 h + t (t = 0..7) of the lane's
//     vector: the B operand of a 32x32x16 MFMA.  Raw bf16 inputs are that
//     operand as loaded; RoPE'd or fp32 inputs are scaled and split into fp16
//     hi + lo parts.  RoPE's pair (i, i + d/2) is steps kb and kb + d/32 of
//     the same lane.
//   * The Walsh-Hadamard transform is H_d = H_{d/32} (x) H32: the A operands
//     are the halves of H32 with the sign flips folded in (and their
//     negations), built once per block in LDS, and output block ob takes
//     step kb with the sign H_{d/32}[ob][kb/2].  Afterwards lane (v, h) holds
//     coordinates 32 ob + 8 (r/4) + 4 h + r%4 in register r of block ob.
//   * Quantiser, residual and packing run on those values; the residual's
//     fp16 hi/lo parts are again a B operand, so the sketch S e of all 32
//     vectors is m/32 row blocks of d/16 MFMA steps, with S read from LDS in
//     the matching coordinate order (laid out by the host).
// Sign correction (TurboESM summary, technical section 2; MODE 1 and 2): the
// sign of every residual coordinate is kept (S = I, m = d) and no gamma, so
// the sketch MFMAs give way to byte-wise sign packing.  MODE 2 also skips the
// rotation (values quantised in their original coordinates): the lane loads
// its output coordinates straight from the input.
// Vector codebooks (FibQuant summary, sections 2.1-2.3; MODE 3): after the
// rotation each lane holds 32 (d = 128) or 16 (d = 64) whole blocks of two
// coordinates (registers r, r + 1 for even r), so the nearest codeword - the
// largest <y, c> - |c|^2 / 2, ties to the smaller index - needs no data
// exchange.  Codebooks of up to 64 codewords look the block's cell up in a
// candidate grid (built by the host, in LDS) and score its four candidates;
// cells with more candidates, blocks off the grid and larger codebooks score
// every codeword.  The indices are packed LSB first, lane half 1's moved up
// by two blocks, and the pair's words merged.
// Blocks are persistent (one resident round, grid-stride over tiles) so each
// block stages its tables in LDS once; tiles run token block, then sequence,
// then head, so a block's four waves encode four heads of the same tokens and
// every user of a token block's RoPE rows runs close together.
//
// Dense form (any d that is a multiple of 64): per-vector norm, then
// Y = U Pi^T and Z = E S^T as MFMA GEMMs over chunks of vectors in the
// caller's workspace, with per-vector quantise and sign-pack kernels between.
#include <hip/hip_runtime.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

struct EncK {
    const void* x;
    int64_t s_seq, s_tok, s_head;
    int32_t n_seq, n_tok, h_kv, tok_offset, L_cap, tok_blocks;
    int64_t n_tiles;
    int32_t rope_stage;  // the block's four waves share their tokens: RoPE rows staged in LDS
    // tile t = (token block * n_seq + seq) * h_kv + head: the tiles that share
    // a token block's RoPE rows (every sequence and head) run close together
    dev::FastDiv div_h, div_seq;  // by h_kv and by n_seq (tile indices are below 2^31)
    // append = 1: one token per (sequence, head); tile t holds vectors
    // [32 t, 32 t + 32) of the n_seq * h_kv list (sequence-major) and the
    // token of sequence b goes to slot pos[b] (its RoPE position too)
    int32_t append;
    const int32_t* pos;
    int32_t rope_npos;
    // paged records (pages != nullptr): page table [n_seq][max_pages] of
    // physical pages of page_size slots, each holding every head's slots
    const int32_t* pages;
    int32_t page_size, max_pages;
    int64_t n_pages;
    dev::FastDiv div_page;
    const float* rope_cos;
    const float* rope_sin;
    const float* sigma;
    const float* levels;
    const float* thresholds;
    const float* sketch_mfma;
    const uint32_t* vq_grid;  // vector codebooks: candidate grid (tq_internal.h), or nullptr
    float vq_inv_cell;
    float* norm;
    float* rnorm;
    uint32_t* codes;
    uint32_t* signs;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// lanes l and l ^ 32 exchange v (v_permlane32_swap): returns {own half's r0, r1}
// where for lanes < 32 r0 = own and r1 = partner, and for lanes >= 32 r0 =
// partner and r1 = own.
struct Swap {
    float r0, r1;
};
__device__ __forceinline__ Swap swap32(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// lanes l and l ^ 32 trade one register each (v_permlane32_swap): afterwards
// the lower lanes hold (own a, upper partner's a) and the upper lanes (lower
// partner's b, own b) - a 2x2 transpose between the lane half and the
// register pair (a, b)
__device__ __forceinline__ void xchg(float& a, float& b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

// Per-coordinate quantiser for 1 and 2 bits, for a symmetric table
// (t_{K-1-k} = -t_k, tau_{K-2-k} = -tau_k, tau_{K/2-1} = 0; the host builds
// the upper half and mirrors it, so this holds exactly).  c = #{j : y >= tau_j}
// is found as the code c' of |y| among the upper thresholds, mirrored for
// y < 0 (there a tie |y| = tau goes to the other side, a decision within
// rounding of the boundary).  Returns the code and the residual
// e = y - t_c = y - sign(y) t_{K/2+c'}.
// pt: the K/2-1 upper thresholds, pl: the K/2 upper levels (scaled).
template <int BITS>
__device__ __forceinline__ uint32_t quantise(float y, const float* pt, const float* pl, float* e) {
    static_assert(BITS <= 2, "3 and 4 bits use the byte-packed path");
    constexpr uint32_t KH = 1u << (BITS - 1);
    uint32_t cp;  // code of |y| among the upper cells
    float lv;
    if constexpr (BITS == 1) {
        cp = 0u;
        lv = pl[0];
    } else {
        const bool m0 = fabsf(y) >= pt[0];
        cp = (uint32_t)m0;
        lv = m0 ? pl[1] : pl[0];
    }
    // e = y - t_c with t_c = sign(y) * lv (one bitfield insert and a subtract)
    *e = y - __builtin_copysignf(lv, y);
    // y >= 0: K/2 + c';  y < 0: K/2 - 1 - c' = (K/2 + c') ^ (K - 1)
    const uint32_t neg = (uint32_t)((int32_t)__float_as_uint(y) >> 31);
    return (KH | cp) ^ (neg & (2u * KH - 1u));
}

// K/2 + c' where c' is the code of a = |y| among the upper cells of a
// symmetric table (pt: the K/2-1 upper thresholds); y's code is this value for
// y >= 0 and its complement in K - 1 bits for y < 0.
// base + m in one carry-in add (the lane mask of m is the carry)
__device__ __forceinline__ uint32_t add_bit(uint32_t base, bool m) {
    uint32_t r;
    uint64_t carry_out;
    asm("v_addc_co_u32 %0, %1, %2, 0, %3" : "=v"(r), "=s"(carry_out) : "v"(base), "s"(__builtin_amdgcn_ballot_w64(m)));
    return r;
}

template <int BITS>
__device__ __forceinline__ uint32_t upper_code(float a, const float* pt) {
    if constexpr (BITS == 3) {
        const bool m1 = a >= pt[1];
        const bool m0 = a >= (m1 ? pt[2] : pt[0]);
        return add_bit(m1 ? 6u : 4u, m0);
    } else {
        static_assert(BITS == 4, "byte-packed codes are used for 3 and 4 bits");
        const bool m2 = a >= pt[3];
        const bool m1 = a >= (m2 ? pt[5] : pt[1]);
        const float t0 = m2 ? pt[4] : pt[0];
        const float t1 = m2 ? pt[6] : pt[2];
        const bool m0 = a >= (m1 ? t1 : t0);
        return add_bit((m2 ? 12u : 8u) + (m1 ? 2u : 0u), m0);
    }
}

// x = hi + lo (fp16 parts: hi = x rounded to nearest, lo = the exact
// remainder x - hi rounded to nearest): x to within 2^-22 |x| while lo stays
// normal.  Per pair: one packed conversion and two mixed-precision FMAs that
// form x - hi exactly before rounding.  The asm operands are the floats as
// stored, so the split cannot be fused with the product that made them.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
    asm volatile("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(hi) : "v"(a), "v"(b));
    asm volatile(
        "v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %0, %1, -1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=&v"(lo)
        : "v"(hi), "v"(a), "v"(b));
}
__device__ __forceinline__ void split_f16(const float* x, half8& hi, half8& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) split_pair(x[2 * q], x[2 * q + 1], h[q], l[q]);
    hi = __builtin_bit_cast(half8, make_uint4(h[0], h[1], h[2], h[3]));
    lo = __builtin_bit_cast(half8, make_uint4(l[0], l[1], l[2], l[3]));
}

// RoPE rows of the 32 tokens of the tile step at `base` (table entries of
// this thread's staging slots), and their store into the LDS buffer
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// buffer resource over [base, base + bytes) (gfx9 word 3: 32-bit elements, no
// swizzle); stores at or past the end are dropped by the hardware
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const uint32_t n = bytes <= 0 ? 0u : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}
// a byte offset past every tile's resource: the store is dropped
constexpr uint32_t kDrop = 0x40000000u;
// N consecutive words at byte offset vo (16-, 8- and 4-byte stores)
template <int N>
__device__ __forceinline__ void store_words(__amdgpu_buffer_rsrc_t r, uint32_t vo, const uint32_t* w) {
    int k = 0;
#pragma unroll
    for (; k + 4 <= N; k += 4)
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[k], w[k + 1], w[k + 2], w[k + 3]}, r, vo + 4u * k, 0, 0);
    if constexpr (N % 4 >= 2) {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[k], w[k + 1]}, r, vo + 4u * k, 0, 0);
        k += 2;
    }
    if constexpr (N % 2 == 1) __builtin_amdgcn_raw_buffer_store_b32(w[k], r, vo + 4u * k, 0, 0);
}

template <int HALF, int NQ>
__device__ __forceinline__ void rope_stage_load(const EncK& p, int64_t base, const int (&tab)[NQ],
                                                const int (&row)[NQ], const int (&c4)[NQ], f32x4 (&pre)[NQ]) {
    const uint32_t r0 = p.div_h.div((uint32_t)base);
    const int tb0 = (int)p.div_seq.div(r0);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const int pos = p.tok_offset + min(tb0 * 32 + row[j], p.n_tok - 1);
        const float* src = (tab[j] ? p.rope_sin : p.rope_cos) + (int64_t)pos * HALF + 4 * c4[j];
        pre[j] = *reinterpret_cast<const f32x4*>(src);
    }
}
template <int RS, int NQ>
__device__ __forceinline__ void rope_stage_store(f32x4* lds, const int (&tab)[NQ], const int (&row)[NQ],
                                                 const int (&c4)[NQ], const f32x4 (&pre)[NQ]) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) lds[((tab[j] * 32 + row[j]) * RS) / 4 + c4[j]] = pre[j];
}

// MODE 0: Hadamard rotation, Gaussian sketch of the residual and gamma;
// 1: Hadamard rotation, sign of each residual coordinate; 2: no rotation,
// sign of each residual coordinate; 3: Hadamard rotation, nearest codeword
// of every two-coordinate block in a vector codebook of 2^BITS codewords.
// GEN: general addressing (appends at per-sequence slots, page tables);
// bulk encodes into contiguous records take the kernel without it, which
// keeps the page-table and slot arguments out of its scalar registers.
// The bulk sign-corrected key encoder at d = 128 needs 170 VGPRs unhinted (two
// waves per SIMD); held to 168 it runs three, with no spills (measured 4 %
// faster).  Every other form keeps the compiler's own allocation.
template <int D, int BITS, int M, bool BF16, bool ROPE, int MODE, bool GEN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu((D == 128 && ROPE && MODE == 1 && !GEN) ? 3
                                                                                                        : 1))) void
encode_had_kernel(EncK p) {
    constexpr bool SGN = MODE == 1 || MODE == 2;
    constexpr bool NOROT = MODE == 2;
    constexpr bool VQ = MODE == 3;
    static_assert(!SGN || M == D, "the sign correction keeps one bit per coordinate");
    static_assert(!VQ || M == 0, "vector codebooks keep no sketch");
    constexpr int HALF = D / 2;
    constexpr int NOB = D / 32;            // 32-coordinate output blocks of H
    constexpr int NKB = D / 16;            // 16-coordinate input steps of the MFMA
    constexpr bool EXACT = BF16 && !ROPE && !NOROT;  // raw bf16 inputs are the MFMA operand as loaded
    constexpr int KH = VQ ? 1 : 1 << (BITS - 1);
    constexpr int CW = VQ ? BITS * D / 64 : BITS * D / 32;  // code words per record
    constexpr int NRB = M / 32;            // sketch row blocks (= sign words)
    constexpr int NP = D / 16;             // sketch K-steps: chunks of 8 values per lane
    constexpr bool SKETCH = M > 0 && !SGN;  // Gaussian sketch on the matrix cores
    constexpr int SKN = SKETCH ? NRB * NP * 2 * 64 : 1;
    // residuals enter the sketch scaled by 2^8 so their fp16 low parts stay normal
    constexpr float ESCALE = 256.0f;
    __shared__ half8 s_sk[SKN];
    // A operands of the Hadamard MFMAs, sign flips folded in: entry [kb][lane]
    // holds H32[lane%32][16(kb%2) + 8(lane/32) + t] * sigma[16kb + 8(lane/32) + t]
    // for t = 0..7 as bf16 (raw bf16 inputs) or fp16 (split inputs) +-1
    // [+A; -A].  With a full-width sketch at d = 128 only +A is kept (-A by
    // sign flips per tile): the tables then stay below half of a CU's LDS, so
    // two blocks fit per CU instead of one.
    constexpr bool NEG_LDS = !(M == D && D == 128) || SGN;
    __shared__ uint4 s_had[NOROT ? 1 : (NEG_LDS ? 2 : 1) * NKB * 64];
    // scaled levels, indexed by code (3 and 4 bits: looked up by K/2 + c')
    __shared__ float s_lvl[16];
    // vector codebook, scaled: {c0, c1, -|c|^2 / 2}; codebooks of up to 64
    // codewords search the candidates of their grid cell
    constexpr int NV = VQ ? 1 << BITS : 1;
    constexpr bool VQGRID = VQ && NV <= kVqGridMaxN;
    __shared__ float4 s_vq[NV];
    __shared__ uint32_t s_grid[VQGRID ? kVqGrid * kVqGrid : 1];

    if constexpr (SKETCH) {
        const half8* src = reinterpret_cast<const half8*>(p.sketch_mfma);
        for (int i = threadIdx.x; i < SKN; i += blockDim.x) s_sk[i] = src[i];
    }
    if (!VQ && threadIdx.x < 16) s_lvl[threadIdx.x] = threadIdx.x < 2 * KH ? p.levels[threadIdx.x] * ESCALE : 0.0f;
    if constexpr (VQ) {
        for (int i = threadIdx.x; i < NV; i += blockDim.x) {
            const float c0 = p.levels[2 * i] * ESCALE, c1 = p.levels[2 * i + 1] * ESCALE;
            s_vq[i] = make_float4(c0, c1, -0.5f * (c0 * c0 + c1 * c1), 0.0f);
        }
    }
    if constexpr (VQGRID) {
        for (int i = threadIdx.x; i < kVqGrid * kVqGrid; i += blockDim.x) s_grid[i] = p.vq_grid[i];
    }
    for (int i = threadIdx.x; i < (NOROT ? 0 : NKB * 64); i += blockDim.x) {
        const int kb = i >> 6, row = i & 31, hh = (i >> 5) & 1;
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t pair = 0;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int t = 2 * q + s;
                const int col = 16 * (kb & 1) + 8 * hh + t;
                const bool neg = ((__popc(row & col) & 1) != 0) != (p.sigma[16 * kb + 8 * hh + t] < 0.0f);
                pair |= ((EXACT ? 0x3F80u : 0x3C00u) | (neg ? 0x8000u : 0u)) << (16 * s);
            }
            w[q] = pair;
        }
        s_had[i] = make_uint4(w[0], w[1], w[2], w[3]);
        if constexpr (NEG_LDS && !NOROT)
            s_had[NKB * 64 + i] = make_uint4(w[0] ^ 0x80008000u, w[1] ^ 0x80008000u, w[2] ^ 0x80008000u, w[3] ^ 0x80008000u);
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int v = lane & 31;
    const int h = lane >> 5;
    // -A of input step kb (ap = +A)
    auto neg_operand = [&](const uint4& ap, int kb, int ln) -> uint4 {
        if constexpr (NEG_LDS && !NOROT) return s_had[NKB * 64 + kb * 64 + ln];
        return make_uint4(ap.x ^ 0x80008000u, ap.y ^ 0x80008000u, ap.z ^ 0x80008000u, ap.w ^ 0x80008000u);
    };

    // upper halves of the symmetric tables, scaled
    float pt[KH > 1 ? KH - 1 : 1], pl[KH];
    if constexpr (!VQ) {
#pragma unroll
        for (int k = 0; k + 1 < KH; ++k) pt[k] = p.thresholds[KH + k] * ESCALE;
#pragma unroll
        for (int k = 0; k < KH; ++k) pl[k] = p.levels[KH + k] * ESCALE;
    }
    // grid coordinates of a scaled block: cell = floor(y * inv_cell / 2^8 + kVqGrid / 2)
    const float vq_gscale = p.vq_inv_cell * (1.0f / ESCALE);
    const float yscale = ESCALE / sqrtf((float)D);

    // RoPE rows of the block's 32 tokens, staged in LDS when the block's four
    // waves encode four heads of the same tokens (h_kv a multiple of 4): the
    // rows of the next tile step are loaded into registers while the current
    // one computes, then written to LDS between two barriers.
    constexpr int RS = HALF + 4;                   // padded row stride (floats)
    constexpr int NQ = 2 * 32 * (HALF / 4) / 256;  // float4 per thread per stage (cos and sin)
    extern __shared__ f32x4 s_rope4[];             // [cos, sin][32 tokens][RS / 4]
    // bulk encodes (!GEN) with RoPE always stage the rows (the launcher sends
    // other head counts to the general kernel), so their loop has no
    // per-lane RoPE loads
    const bool stage = ROPE && (!GEN || p.rope_stage != 0);
    int st_table[NQ], st_row[NQ], st_c4[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const int q = threadIdx.x + 256 * j;
        st_table[j] = q / (32 * (HALF / 4));
        const int rem = q % (32 * (HALF / 4));
        st_row[j] = rem / (HALF / 4);
        st_c4[j] = rem % (HALF / 4);
    }
    const int64_t blk_stride = (int64_t)gridDim.x * 4;
    int64_t base = (int64_t)blockIdx.x * 4;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // wave (scalar)
    // element offset of this lane's input vector in tile t; lanes past the
    // last token read the last token instead (an MFMA column only feeds its
    // own vector, and these vectors are not stored)
    auto input_offset = [&](int64_t t) -> int64_t {
        if (GEN && p.append) {
            const int64_t idx = min(t * 32 + v, (int64_t)p.n_seq * p.h_kv - 1);
            const uint32_t b = p.div_h.div((uint32_t)idx);
            return (int64_t)b * p.s_seq + (int64_t)((uint32_t)idx - b * (uint32_t)p.h_kv) * p.s_head;
        }
        const uint32_t r = p.div_h.div((uint32_t)t);
        const int hd = (int)((uint32_t)t - r * (uint32_t)p.h_kv);
        const uint32_t tq_ = p.div_seq.div(r);
        const uint32_t sq = r - tq_ * (uint32_t)p.n_seq;
        const int tbk = (int)tq_;
        return (int64_t)sq * p.s_seq + (int64_t)min(tbk * 32 + v, p.n_tok - 1) * p.s_tok + (int64_t)hd * p.s_head;
    };
    // record of slot t of (sequence b, head hd), or -1 for a slot outside the
    // cache (or behind a page-table entry outside the pool): such a vector is
    // encoded but not stored
    auto record_of = [&](int b, int hd, int64_t t) -> int64_t {
        if (GEN && p.pages) {
            if (t < 0 || t >= (int64_t)p.max_pages * p.page_size) return -1;
            const uint32_t j = p.div_page.div((uint32_t)t);
            const int32_t pg = p.pages[(int64_t)b * p.max_pages + j];
            if (pg < 0 || pg >= p.n_pages) return -1;
            return ((int64_t)pg * p.h_kv + hd) * p.page_size + (t - (int64_t)j * p.page_size);
        }
        if (t < 0 || t >= p.L_cap) return -1;
        return ((int64_t)b * p.h_kv + hd) * p.L_cap + t;
    };
    // RoPE keys run at two waves per SIMD whatever their register count, so
    // their next tile's bf16 inputs are loaded while this tile is quantised
    // (vector codebooks keep neither prefetch: their search needs the
    // registers, and a third wave per SIMD hides the loads instead)
    constexpr bool PREFETCH = ROPE && BF16 && D == 128 && !NOROT && !VQ;
    constexpr bool ROW_PREFETCH = !VQ;  // next step's RoPE rows in registers during the tile
    uint4 nxt[PREFETCH ? NKB : 1];
    if constexpr (PREFETCH) {
        // bulk encodes load a tile past the last as the last (unused), so the
        // load is unconditional
        const int64_t t0 = GEN ? base + wv : min(base + wv, p.n_tiles - 1);
        if (!GEN || t0 < p.n_tiles) {
            const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.x) + input_offset(t0));
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) nxt[kb] = src[2 * kb + h];
        }
    }
    // the first step's RoPE rows (after the first inputs are requested: the
    // rows' wait then covers them, and the loop starts with nothing in
    // flight, as each iteration ends with only its prefetches and stores)
    if (stage && base < p.n_tiles) {
        f32x4 pre[NQ];
        rope_stage_load<HALF, NQ>(p, base, st_table, st_row, st_c4, pre);
        rope_stage_store<RS, NQ>(s_rope4, st_table, st_row, st_c4, pre);
    }
    __syncthreads();
    // the loop bound is the same for the whole block (barriers inside)
    for (; base < p.n_tiles; base += blk_stride) {
      const int64_t tile = base + wv;
      const bool live = tile < p.n_tiles;
      // Bulk encodes run every wave through the tile body - a wave past the
      // last tile computes on the last and stores nothing - and issue their
      // loads and stores unconditionally: with no memory operation behind a
      // branch, the compiler's in-order count of outstanding operations stays
      // exact and a wait for the prefetched inputs waits for nothing else.
      const int64_t ctile = GEN ? tile : min(tile, p.n_tiles - 1);
      // the next step's rows, in flight during this step's quantiser (loaded
      // once this tile's own input registers are free; bulk encodes reload
      // the last step's rows at the last step)
      f32x4 pre[NQ];
      const bool prefetch = ROW_PREFETCH && stage && (!GEN || base + blk_stride < p.n_tiles);
      const int64_t pbase = GEN ? base + blk_stride : min(base + blk_stride, p.n_tiles - 1);
      if (GEN && !live && prefetch) rope_stage_load<HALF, NQ>(p, pbase, st_table, st_row, st_c4, pre);
      if (!GEN || live) {
        // the lane's vector: sequence, head, cache slot, RoPE row (a valid
        // table row for every lane) and whether it is stored.  Computed at
        // the start for the RoPE row, and again from the lane's index at the
        // stores, so the record address holds no registers in between.
        struct Loc {
            int seq, head, rpos;
            int64_t slot;
            bool valid;
        };
        auto locate = [&](int vl) -> Loc {
            Loc L;
            if (GEN && p.append) {
                const int64_t idx = ctile * 32 + vl;
                const int64_t nv = (int64_t)p.n_seq * p.h_kv;
                const uint32_t bq = p.div_h.div((uint32_t)min(idx, nv - 1));
                L.seq = (int)bq;
                L.head = (int)((uint32_t)min(idx, nv - 1) - bq * (uint32_t)p.h_kv);
                L.slot = p.pos[L.seq];
                L.valid = idx < nv;
                L.rpos = (int)min(max(L.slot, (int64_t)0), (int64_t)max(p.rope_npos - 1, 0));
            } else {
                const uint32_t r = p.div_h.div((uint32_t)ctile);
                L.head = (int)((uint32_t)ctile - r * (uint32_t)p.h_kv);
                const uint32_t tbq = p.div_seq.div(r);
                L.seq = (int)(r - tbq * (uint32_t)p.n_seq);
                const int token = (int)tbq * 32 + vl;
                L.valid = token < p.n_tok;
                L.slot = (int64_t)p.tok_offset + token;
                L.rpos = p.tok_offset + (L.valid ? token : 0);
            }
            return L;
        };
        // record index and store flag, at the stores (the lane index passes
        // through an empty asm so that the address is recomputed there, not
        // carried from the start)
        auto record = [&](int64_t* n_out) -> bool {
            int vl = v;
            asm volatile("" : "+v"(vl));
            const Loc L = locate(vl);
            const int64_t rec = record_of(L.seq, L.head, L.slot);
            *n_out = rec;
            return L.valid && rec >= 0;
        };
        const int rpos = locate(v).rpos;
        // bulk encodes: the tile's vectors are 32 consecutive slots of one
        // (sequence, head), so one buffer resource per plane spans the records
        // the tile stores (none for a tile past the last); stores of vectors
        // past the last token, and of the other lane half's words, fall
        // outside it or go to kDrop
        __amdgpu_buffer_rsrc_t o_codes = make_rsrc(nullptr, 0), o_norm = o_codes, o_rnorm = o_codes, o_signs = o_codes;
        if constexpr (!GEN) {
            const uint32_t r = p.div_h.div((uint32_t)ctile);
            const int hd = (int)((uint32_t)ctile - r * (uint32_t)p.h_kv);
            const uint32_t tbq = p.div_seq.div(r);
            const int sq = (int)(r - tbq * (uint32_t)p.n_seq);
            const int tok0 = (int)tbq * 32;
            const int64_t cnt = live ? min(32, p.n_tok - tok0) : 0;
            const int64_t rec0 = ((int64_t)sq * p.h_kv + hd) * p.L_cap + p.tok_offset + tok0;
            o_codes = make_rsrc(p.codes + rec0 * CW, cnt * CW * 4);
            o_norm = make_rsrc(p.norm + rec0, cnt * 4);
            if constexpr (M > 0 && !SGN) o_rnorm = make_rsrc(p.rnorm + rec0, cnt * 4);
            if constexpr (M > 0) o_signs = make_rsrc(p.signs + rec0 * (M / 32), cnt * (M / 32) * 4);
        }

        floatx16 acc[NOB];
        float nu, scale;
        if constexpr (NOROT) {
            // register r of block ob holds coordinate 32 ob + 8 (r/4) + 4 h + r%4
            // (the layout the Hadamard MFMAs leave): four contiguous inputs per
            // (ob, r/4), loaded as they are
            float xs[NOB][16];
            const int64_t off = input_offset(ctile);
#pragma unroll
            for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c0 = 32 * ob + 8 * g + 4 * h;
                    if constexpr (BF16) {
                        const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.x) + off + c0);
                        xs[ob][4 * g] = bf16_lo(w.x);
                        xs[ob][4 * g + 1] = bf16_hi(w.x);
                        xs[ob][4 * g + 2] = bf16_lo(w.y);
                        xs[ob][4 * g + 3] = bf16_hi(w.y);
                    } else {
                        const f32x4 w = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.x) + off + c0);
#pragma unroll
                        for (int j = 0; j < 4; ++j) xs[ob][4 * g + j] = w[j];
                    }
                }
            float ss = 0.0f;
#pragma unroll
            for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                for (int r = 0; r < 16; ++r) ss = fmaf(xs[ob][r], xs[ob][r], ss);
            {
                const Swap sw = swap32(ss);
                ss = sw.r0 + sw.r1;
            }
            nu = sqrtf(ss);
            scale = nu > 0.0f ? ESCALE / nu : 0.0f;
            // y = 2^8 RoPE(x) / nu; + 0 turns a -0 into +0, whose code is that of 0
            if constexpr (ROPE) {
                // pair (i, i + D/2) is blocks ob and ob + NOB/2 at the same register
#pragma unroll
                for (int ob = 0; ob < NOB / 2; ++ob)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int c0 = 32 * ob + 8 * g + 4 * h;
                        f32x4 cc, sn;
                        if (stage) {
                            cc = s_rope4[(v * RS + c0) / 4];
                            sn = s_rope4[((32 + v) * RS + c0) / 4];
                        } else {
                            const int64_t ro = (int64_t)rpos * HALF + c0;
                            cc = *reinterpret_cast<const f32x4*>(p.rope_cos + ro);
                            sn = *reinterpret_cast<const f32x4*>(p.rope_sin + ro);
                        }
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float cs = cc[j] * scale, sv = sn[j] * scale;
                            const float lo = xs[ob][4 * g + j], hi = xs[ob + NOB / 2][4 * g + j];
                            acc[ob][4 * g + j] = fmaf(lo, cs, -(hi * sv)) + 0.0f;
                            acc[ob + NOB / 2][4 * g + j] = fmaf(hi, cs, lo * sv) + 0.0f;
                        }
                    }
            } else {
#pragma unroll
                for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[ob][r] = fmaf(xs[ob][r], scale, 0.0f);
            }
        } else {
        // B operands: input step kb is coordinates 16kb + 8h + t (t = 0..7)
        // of this lane's vector
        uint4 raw[BF16 ? NKB : 1];
        float xv[BF16 ? 1 : NKB][8];
        float ss = 0.0f;
        if constexpr (BF16) {
            if constexpr (PREFETCH) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) raw[kb] = nxt[kb];
            } else {
                const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.x) + input_offset(ctile));
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) raw[kb] = src[2 * kb + h];
            }
            // nu^2 from the bf16 pairs (RoPE keeps the norm)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, raw[kb].x),
                                                     __builtin_bit_cast(bf16x2, raw[kb].x), ss, false);
                ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, raw[kb].y),
                                                     __builtin_bit_cast(bf16x2, raw[kb].y), ss, false);
                ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, raw[kb].z),
                                                     __builtin_bit_cast(bf16x2, raw[kb].z), ss, false);
                ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, raw[kb].w),
                                                     __builtin_bit_cast(bf16x2, raw[kb].w), ss, false);
            }
        } else {
            const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.x) + input_offset(ctile));
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const f32x4 a = src[4 * kb + 2 * h];
                const f32x4 b = src[4 * kb + 2 * h + 1];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    xv[kb][u] = a[u];
                    xv[kb][4 + u] = b[u];
                }
            }
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int t = 0; t < 8; ++t) ss = fmaf(xv[kb][t], xv[kb][t], ss);
        }
        {
            const Swap sw = swap32(ss);
            ss = sw.r0 + sw.r1;
        }
        nu = sqrtf(ss);
        // maps H(sigma * x) to 2^8 * Pi (x / nu)
        scale = nu > 0.0f ? yscale / nu : 0.0f;

        // Walsh-Hadamard transform as MFMAs: H_D = H_{D/32} (x) H32, so output
        // block ob takes input step kb with the sign H_{D/32}[ob][kb/2].
        // Output block ob, register r of this lane = coordinate
        // 32 ob + 8 (r/4) + 4 h + r%4.
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[ob][q] = 0.0f;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (EXACT) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const uint4 ap = s_had[kb * 64 + lane];
                const uint4 an = neg_operand(ap, kb, lane);
#pragma unroll
                for (int ob = 0; ob < NOB; ++ob) {
                    const uint4 a = (__builtin_popcount(ob & (kb >> 1)) & 1) ? an : ap;
                    acc[ob] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                                     __builtin_bit_cast(bf16x8, raw[kb]), acc[ob], 0, 0, 0);
                }
            }
        } else {
            // split inputs, one RoPE pair of steps at a time (pair (i, i + D/2)
            // is steps kb and kb + NKB/2 at the same t): RoPE, the scale, fp16
            // hi + lo parts, then both parts through the MFMAs
#pragma unroll
            for (int kp = 0; kp < NKB / 2; ++kp) {
                float xl[8], xh[8];
                if constexpr (BF16) {
                    const uint32_t wl[4] = {raw[kp].x, raw[kp].y, raw[kp].z, raw[kp].w};
                    const uint4 rh = raw[kp + NKB / 2];
                    const uint32_t wh[4] = {rh.x, rh.y, rh.z, rh.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        xl[2 * q] = bf16_lo(wl[q]);
                        xl[2 * q + 1] = bf16_hi(wl[q]);
                        xh[2 * q] = bf16_lo(wh[q]);
                        xh[2 * q + 1] = bf16_hi(wh[q]);
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        xl[t] = xv[kp][t];
                        xh[t] = xv[kp + NKB / 2][t];
                    }
                }
                if constexpr (ROPE) {
                    f32x4 cc[2], sn[2];
                    if (stage) {
#pragma unroll
                        for (int c = 0; c < 2; ++c) {
                            cc[c] = s_rope4[(v * RS + 16 * kp + 8 * h) / 4 + c];
                            sn[c] = s_rope4[((32 + v) * RS + 16 * kp + 8 * h) / 4 + c];
                        }
                    } else {
                        const int64_t ro = (int64_t)rpos * HALF + 16 * kp + 8 * h;
                        const f32x4* cp = reinterpret_cast<const f32x4*>(p.rope_cos + ro);
                        const f32x4* sp = reinterpret_cast<const f32x4*>(p.rope_sin + ro);
#pragma unroll
                        for (int c = 0; c < 2; ++c) {
                            cc[c] = cp[c];
                            sn[c] = sp[c];
                        }
                    }
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const float cs = cc[t >> 2][t & 3] * scale, s = sn[t >> 2][t & 3] * scale;
                        const float lo = xl[t], hi = xh[t];
                        xl[t] = fmaf(lo, cs, -(hi * s));
                        xh[t] = fmaf(hi, cs, lo * s);
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        xl[t] *= scale;
                        xh[t] *= scale;
                    }
                }
#pragma unroll
                for (int side = 0; side < 2; ++side) {
                    const int kb = kp + side * (NKB / 2);
                    const float* xs = side ? xh : xl;
                    half8 bhi, blo;
                    split_f16(xs, bhi, blo);
                    const uint4 ap = s_had[kb * 64 + lane];
                    const uint4 an = neg_operand(ap, kb, lane);
#pragma unroll
                    for (int ob = 0; ob < NOB; ++ob) {
                        const half8 a = __builtin_bit_cast(half8, (__builtin_popcount(ob & (kb >> 1)) & 1) ? an : ap);
                        acc[ob] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bhi, acc[ob], 0, 0, 0);
                        acc[ob] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, blo, acc[ob], 0, 0, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        }  // rotation
        __builtin_amdgcn_sched_barrier(0);
        if (prefetch) rope_stage_load<HALF, NQ>(p, pbase, st_table, st_row, st_c4, pre);
        if constexpr (PREFETCH) {
            const int64_t tn = GEN ? tile + blk_stride : min(tile + blk_stride, p.n_tiles - 1);
            if (!GEN || tn < p.n_tiles) {
                const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.x) + input_offset(tn));
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) nxt[kb] = src[2 * kb + h];
            }
        }

        if constexpr (VQ) {
            // block j = 16 ob + 4 (r/4) + 2 h + (r%4)/2 is registers r, r + 1
            // (r even); indices are packed at lane half 0's positions (h = 0)
            uint32_t cw[CW];
#pragma unroll
            for (int w = 0; w < CW; ++w) cw[w] = 0u;
            // (pairs one at a time: batching the cells' grid reads costs
            // registers and occupancy, which the values' encoder needs more)
#pragma unroll
            for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float y0 = EXACT ? fmaf(acc[ob][r], scale, 0.0f) : acc[ob][r];
                    const float y1 = EXACT ? fmaf(acc[ob][r + 1], scale, 0.0f) : acc[ob][r + 1];
                    // the nearest codeword: the first maximum of <y, c> - |c|^2 / 2
                    // over the cell's candidates, or over the whole codebook
                    float bs = -INFINITY;
                    uint32_t bi = 0u;
                    bool full = true;
                    if constexpr (VQGRID) {
                        const int ix = (int)floorf(fmaf(y0, vq_gscale, 0.5f * kVqGrid));
                        const int iy = (int)floorf(fmaf(y1, vq_gscale, 0.5f * kVqGrid));
                        const bool in = ((ix | iy) & ~(kVqGrid - 1)) == 0;
                        const uint32_t cw0 = s_grid[in ? (iy << kVqGridLog) | ix : 0];
                        // a flagged cell (byte 0 = 0xFF) searches everything;
                        // its candidate reads stay at codeword 0
                        full = !in || (cw0 & 0xFFu) == 0xFFu;
                        const uint32_t cand = full ? 0u : cw0;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const uint32_t c = (cand >> (8 * q)) & 0xFFu;
                            const float4 cv = s_vq[c];
                            const float sc = fmaf(cv.x, y0, fmaf(cv.y, y1, cv.z));
                            if (sc > bs) {
                                bs = sc;
                                bi = c;
                            }
                        }
                    }
                    if (full) {
                        bs = -INFINITY;
                        for (int c = 0; c < NV; ++c) {
                            const float4 cv = s_vq[c];
                            const float sc = fmaf(cv.x, y0, fmaf(cv.y, y1, cv.z));
                            if (sc > bs) {
                                bs = sc;
                                bi = (uint32_t)c;
                            }
                        }
                    }
                    const int o = (16 * ob + 4 * (r / 4) + (r % 4) / 2) * BITS;
                    cw[o >> 5] |= bi << (o & 31);
                    if ((o & 31) + BITS > 32) cw[(o >> 5) + 1] |= bi >> (32 - (o & 31));
                }
            // lane half 1's blocks sit two blocks (2 BITS bits) higher
            if (h) {
#pragma unroll
                for (int w = CW - 1; w > 0; --w) cw[w] = (cw[w] << (2 * BITS)) | (cw[w - 1] >> (32 - 2 * BITS));
                cw[0] <<= 2 * BITS;
            }
            // merge the pair's bits; lane half h stores its share of the words
            constexpr int HW = (CW + 1) / 2;
#pragma unroll
            for (int w = 0; w < CW; ++w) {
                const Swap sw = swap32(__uint_as_float(cw[w]));
                cw[w] = __float_as_uint(sw.r0) | __float_as_uint(sw.r1);
            }
            if constexpr (!GEN) {
                const uint32_t vo = (uint32_t)(v * CW) * 4u;
                if constexpr (CW % 8 == 0) {
                    store_words<HW>(o_codes, vo + 4u * (h * HW), cw + h * HW);
                } else {
#pragma unroll
                    for (int w = 0; w < CW; ++w)
                        __builtin_amdgcn_raw_buffer_store_b32(cw[w], o_codes, (w >= HW) == (h == 1) ? vo + 4u * w : kDrop, 0, 0);
                }
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(nu), o_norm, h == 0 ? 4u * v : kDrop, 0, 0);
            } else {
            int64_t n;
            const bool valid = record(&n);
            if (valid) {
                uint32_t* dst = p.codes + n * CW;
                if constexpr (CW % 8 == 0) {
#pragma unroll
                    for (int k = 0; k < HW / 4; ++k) {
                        const int w0 = h * HW + 4 * k;
                        reinterpret_cast<uint4*>(dst + h * HW)[k] = make_uint4(cw[w0], cw[w0 + 1], cw[w0 + 2], cw[w0 + 3]);
                    }
                } else {
#pragma unroll
                    for (int w = 0; w < CW; ++w)
                        if ((w >= HW) == (h == 1)) dst[w] = cw[w];
                }
                if (h == 0) p.norm[n] = nu;
            }
            }
        } else {
            // per 8-value chunk pc (block pc/2, registers 8(pc%2)..+7): quantise,
            // residual, pack, and feed the residual's fp16 hi/lo parts to the
            // sketch MFMAs.  Codes are packed at lane half 0's positions; lane
            // half 1's are moved into place afterwards.
            uint32_t cw[CW];
    #pragma unroll
            for (int w = 0; w < CW; ++w) cw[w] = 0u;
            float gg = 0.0f;
            floatx16 sacc[SKETCH ? NRB : 1];
    #pragma unroll
            for (int rb = 0; rb < (SKETCH ? NRB : 0); ++rb)
    #pragma unroll
                for (int q = 0; q < 16; ++q) sacc[rb][q] = 0.0f;
            // sign correction: per block, the negative-residual flags of the lane's
            // coordinates, byte a = coordinates 8a + 4h + 0..3 in bits 0..3
            uint32_t wsg[SGN ? NOB : 1];
    #pragma unroll
            for (int ob = 0; ob < (SGN ? NOB : 1); ++ob) wsg[ob] = 0u;
    #pragma unroll
            for (int pc = 0; pc < NP; ++pc) {
                const int ob = pc >> 1, hf = pc & 1;
                float e[8];
                if constexpr (BITS >= 3) {
                    // byte-packed codes: the four codes of a group (t = 4g..4g+3,
                    // one 8-coordinate row a = 2hf + g) as bytes of P, then the
                    // negative coordinates complemented at once through a byte
                    // mask built from the four sign bits (v_perm byte selects)
                    float yv[8];
                    uint32_t xu[8];
    #pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        // + 0: a zero vector's -0 coordinates count as +0 (code of y = 0)
                        yv[t] = EXACT ? fmaf(acc[ob][8 * hf + t], scale, 0.0f) : acc[ob][8 * hf + t];
                        xu[t] = upper_code<BITS>(fabsf(yv[t]), pt);
                    }
    #pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        e[t] = yv[t] - __builtin_copysignf(s_lvl[xu[t]], yv[t]);
                        if constexpr (!SGN) gg = fmaf(e[t], e[t], gg);
                    }
    #pragma unroll
                    for (int g = 0; g < 2; ++g) {
                        const int t0 = 4 * g, a = 2 * hf + g;
                        const uint32_t P = xu[t0] | (xu[t0 + 1] << 8) | (xu[t0 + 2] << 16) | (xu[t0 + 3] << 24);
                        const uint32_t Mk = __builtin_amdgcn_perm(__float_as_uint(yv[t0 + 1]), __float_as_uint(yv[t0]), 0x0C0C0B09u) |
                                            __builtin_amdgcn_perm(__float_as_uint(yv[t0 + 3]), __float_as_uint(yv[t0 + 2]), 0x0B090C0Cu);
                        const uint32_t C = P ^ (Mk & (0x01010101u * (2u * KH - 1u)));
                        if constexpr (BITS == 3) {
                            // lane half 0 positions: rows 0-2 fill bits 0-2 of every
                            // byte of word a; row 3 puts its low bits at 6-7 of word 0
                            // and its high bit at 6 of word 2
                            if (a < 3) {
                                cw[3 * ob + a] |= C;
                            } else {
                                cw[3 * ob] |= (C & 0x03030303u) << 6;
                                cw[3 * ob + 2] |= (C & 0x04040404u) << 4;
                            }
                        } else {
                            // nibble b of word 4 ob + a
                            const uint32_t t2 = C | (C >> 4);
                            cw[4 * ob + a] |= __builtin_amdgcn_perm(t2, t2, 0x0C0C0200u);
                        }
                    }
                } else {
    #pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        // + 0: a zero vector's -0 coordinates count as +0 (code of y = 0)
                        const float y = EXACT ? fmaf(acc[ob][8 * hf + t], scale, 0.0f) : acc[ob][8 * hf + t];
                        const uint32_t code = quantise<BITS>(y, pt, pl, &e[t]);
                        if constexpr (!SGN) gg = fmaf(e[t], e[t], gg);
                        dev::code_put(cw, dev::code_loc(32 * ob + 8 * (2 * hf + (t >> 2)) + (t & 3), BITS), BITS, code);
                    }
                }
                if constexpr (SGN) {
                    // the four flags of group g as bytes 0xFF / 0x00 (v_perm sign
                    // selects), one bit kept per byte, summed into byte 3 by a
                    // multiply and moved to byte a = 2 hf + g of the block's word
    #pragma unroll
                    for (int g = 0; g < 2; ++g) {
                        const int a = 2 * hf + g;
                        const uint32_t f0 = __float_as_uint(e[4 * g]), f1 = __float_as_uint(e[4 * g + 1]);
                        const uint32_t f2 = __float_as_uint(e[4 * g + 2]), f3 = __float_as_uint(e[4 * g + 3]);
                        const uint32_t sb = (__builtin_amdgcn_perm(f1, f0, 0x0C0C0B09u) | __builtin_amdgcn_perm(f3, f2, 0x0B090C0Cu)) &
                                            0x08040201u;
                        wsg[ob] = __builtin_amdgcn_perm(sb * 0x01010101u, wsg[ob],
                                                        (0x03020100u & ~(0xFFu << (8 * a))) | (0x07u << (8 * a)));
                    }
                }
                if constexpr (SKETCH) {
                    half8 ehi, elo;
                    split_f16(e, ehi, elo);
    #pragma unroll
                    for (int rb = 0; rb < NRB; ++rb) {
                        const half8 shi = s_sk[((rb * NP + pc) * 2 + 0) * 64 + lane];
                        sacc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(shi, ehi, sacc[rb], 0, 0, 0);
                    }
    #pragma unroll
                    for (int rb = 0; rb < NRB; ++rb) {
                        const half8 shi = s_sk[((rb * NP + pc) * 2 + 0) * 64 + lane];
                        sacc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(shi, elo, sacc[rb], 0, 0, 0);
                    }
    #pragma unroll
                    for (int rb = 0; rb < NRB; ++rb) {
                        const half8 slo = s_sk[((rb * NP + pc) * 2 + 1) * 64 + lane];
                        sacc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(slo, ehi, sacc[rb], 0, 0, 0);
                    }
                }
                // (per-coordinate packing: the chunk's codes are merged into the
                // words here, not at the final store, which would keep every
                // compare mask alive)
                if constexpr (BITS < 3) {
    #pragma unroll
                    for (int w = 0; w < CW; ++w) asm volatile("" : "+v"(cw[w]));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            {
                const Swap sw = swap32(gg);
                gg = sw.r0 + sw.r1;
            }
            const float gamma = sqrtf(gg) * (1.0f / ESCALE);

            // lane half 1's coordinates are 4 above lane half 0's in every block of
            // 8: for b = 1, 2, 4 its codes sit 4b bits higher in the same words.
            // For b = 3 they sit 3 bits higher in each byte, except the group's
            // last four, whose low bits go to word 1 (not 0) at the same place
            // and whose high bit sits one bit higher in word 2.
            if constexpr (BITS == 3) {
    #pragma unroll
                for (int g = 0; g < NOB; ++g) {
                    const uint32_t w0 = cw[3 * g], w1 = cw[3 * g + 1], w2 = cw[3 * g + 2];
                    cw[3 * g] = h ? (w0 & 0x07070707u) << 3 : w0;
                    cw[3 * g + 1] = h ? (w1 << 3) | (w0 & 0xC0C0C0C0u) : w1;
                    cw[3 * g + 2] = h ? ((w2 & 0x07070707u) << 3) | ((w2 & 0x40404040u) << 1) : w2;
                }
            } else {
                const int sh = h * 4 * BITS;
    #pragma unroll
                for (int w = 0; w < CW; ++w) cw[w] <<= sh;
            }
            // merge the lane pair's bits: lane half h keeps words [h CW/2, (h+1) CW/2)
    #pragma unroll
            for (int k = 0; k < CW / 2; ++k) {
                float a = __uint_as_float(cw[k]), b = __uint_as_float(cw[k + CW / 2]);
                xchg(a, b);
                cw[k] = __float_as_uint(a) | __float_as_uint(b);
            }

            int64_t n = 0;
            bool valid = false;
            if constexpr (!GEN) {
                store_words<CW / 2>(o_codes, (uint32_t)(v * CW + h * (CW / 2)) * 4u, cw);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(nu), o_norm, h == 0 ? 4u * v : kDrop, 0, 0);
                if constexpr (SKETCH)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gamma), o_rnorm, h == 1 ? 4u * v : kDrop, 0, 0);
            } else {
                valid = record(&n);
                if (valid) {
                    uint32_t* dst = p.codes + n * CW + h * (CW / 2);
    #pragma unroll
                    for (int k = 0; k < CW / 2; ++k) dst[k] = cw[k];
                    if (h == 0) p.norm[n] = nu;
                    else if (SKETCH) p.rnorm[n] = gamma;
                }
            }

            if constexpr (SGN) {
                // a set flag is a negative residual: complement, place lane half
                // 1's nibbles 4 bits up, merge the pair; lane half h stores the
                // blocks of its parity
    #pragma unroll
                for (int ob = 0; ob < NOB; ++ob) {
                    uint32_t wb = (~wsg[ob] & 0x0F0F0F0Fu) << (4 * h);
                    const Swap sw = swap32(__uint_as_float(wb));
                    wb = __float_as_uint(sw.r0) | __float_as_uint(sw.r1);
                    if constexpr (!GEN)
                        __builtin_amdgcn_raw_buffer_store_b32(wb, o_signs, (ob & 1) == h ? 4u * (v * NOB + ob) : kDrop, 0, 0);
                    else if (valid && (ob & 1) == h)
                        p.signs[n * NOB + ob] = wb;
                }
            }
            if constexpr (SKETCH) {
                // D[i][j]: j = lane % 32 (vector), i = 8*(r/4) + 4*(lane/32) + r%4 (sketch row)
    #pragma unroll
                for (int rb = 0; rb < NRB; ++rb) {
                    // per byte b: the sign bits of rows 8b + 4h + 0..3 as 0xFF/0x00
                    // bytes (v_perm sign selects), one bit kept per byte, gathered
                    // into byte 3 by a multiply and moved to byte b; a set bit is
                    // a negative value, so the word is complemented at the end
                    uint32_t wb = 0;
    #pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const uint32_t f0 = __float_as_uint(sacc[rb][4 * b]), f1 = __float_as_uint(sacc[rb][4 * b + 1]);
                        const uint32_t f2 = __float_as_uint(sacc[rb][4 * b + 2]), f3 = __float_as_uint(sacc[rb][4 * b + 3]);
                        const uint32_t sb = (__builtin_amdgcn_perm(f1, f0, 0x0C0C0B09u) | __builtin_amdgcn_perm(f3, f2, 0x0B090C0Cu)) &
                                            0x08040201u;
                        // byte 3 of the product = bits 0..3; v_perm puts it at byte b of wb
                        wb = __builtin_amdgcn_perm(sb * 0x01010101u, wb, (0x03020100u & ~(0xFFu << (8 * b))) | (0x07u << (8 * b)));
                    }
                    wb = (~wb & 0x0F0F0F0Fu) << (4 * h);
                    const Swap sw = swap32(__uint_as_float(wb));
                    wb = __float_as_uint(sw.r0) | __float_as_uint(sw.r1);
                    if constexpr (!GEN)
                        __builtin_amdgcn_raw_buffer_store_b32(wb, o_signs, (rb & 1) == h ? 4u * (v * NRB + rb) : kDrop, 0, 0);
                    else if (valid && (rb & 1) == h)
                        p.signs[n * NRB + rb] = wb;
                }
            }
        }
      }
      if (stage) {
          __syncthreads();  // every wave is done with the current rows
          if (base + blk_stride < p.n_tiles) {
              if constexpr (!ROW_PREFETCH) rope_stage_load<HALF, NQ>(p, pbase, st_table, st_row, st_c4, pre);
              rope_stage_store<RS, NQ>(s_rope4, st_table, st_row, st_c4, pre);
          }
          __syncthreads();
      }
    }
}

// ---------------------------------------------------------------- dense form
struct DenseK {
    const void* x;
    int64_t s_seq, s_tok, s_head;
    int32_t n_tok, h_kv, tok_offset, L_cap, d, m, bits;
    int32_t block;  // vector codebooks: coordinates per block (levels holds the N x block codewords)
    int64_t start, count;
    int32_t bf16;
    const float* rope_cos;
    const float* rope_sin;
    const float* levels;
    const float* thresholds;
    float* U;  // [count][d]  unit vectors, later residuals
    float* Y;  // [count][d]  rotated
    float* Z;  // [count][m]  sketch values
    float* norm;
    float* rnorm;
    uint32_t* codes;
    uint32_t* signs;
};

__device__ __forceinline__ int64_t dense_record(const DenseK& p, int64_t vi, int64_t* src_off, int* tok) {
    const int head = (int)(vi % p.h_kv);
    const int64_t r = vi / p.h_kv;
    const int t = (int)(r % p.n_tok);
    const int64_t seq = r / p.n_tok;
    *tok = t;
    *src_off = seq * p.s_seq + (int64_t)t * p.s_tok + (int64_t)head * p.s_head;
    return (seq * p.h_kv + head) * p.L_cap + p.tok_offset + t;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// one wave per vector: RoPE (if tables), nu, u = x / nu into U
__global__ __launch_bounds__(256) void dense_prep_kernel(DenseK p) {
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * 4;
    const int half = p.d / 2;
    for (int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); i < p.count; i += stride) {
        int64_t off;
        int tok;
        const int64_t n = dense_record(p, p.start + i, &off, &tok);
        float ss = 0.0f;
        float* u = p.U + i * p.d;
        for (int c = lane; c < half; c += 64) {
            float a, b;
            if (p.bf16) {
                const uint16_t* s = static_cast<const uint16_t*>(p.x) + off;
                a = __uint_as_float((uint32_t)s[c] << 16);
                b = __uint_as_float((uint32_t)s[c + half] << 16);
            } else {
                const float* s = static_cast<const float*>(p.x) + off;
                a = s[c];
                b = s[c + half];
            }
            if (p.rope_cos) {
                const int64_t pos = p.tok_offset + tok;
                const float cs = p.rope_cos[pos * half + c], sn = p.rope_sin[pos * half + c];
                const float a2 = a * cs - b * sn;
                const float b2 = b * cs + a * sn;
                a = a2;
                b = b2;
            }
            u[c] = a;
            u[c + half] = b;
            ss = fmaf(a, a, fmaf(b, b, ss));
        }
        ss = wave_sum(ss);
        const float nu = sqrtf(ss);
        const float inv = nu > 0.0f ? 1.0f / nu : 0.0f;
        for (int c = lane; c < p.d; c += 64) u[c] = u[c] * inv;
        if (lane == 0) p.norm[n] = nu;
    }
}

// one wave per vector: codes from Y (assembled in LDS), residual into U, gamma
constexpr int kMaxCodeWords = 4 * 4096 / 32;
__global__ __launch_bounds__(256) void dense_quant_kernel(DenseK p) {
    __shared__ uint32_t words[4][kMaxCodeWords];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int K = 1 << p.bits;
    const int cw = p.bits * p.d / 32;
    float lv[16], th[15];
    for (int k = 0; k < 16; ++k) lv[k] = k < K ? p.levels[k] : 0.0f;
    for (int k = 0; k < 15; ++k) th[k] = k < K - 1 ? p.thresholds[k] : INFINITY;
    const int64_t stride = (int64_t)gridDim.x * 4;
    // the loop bound is the same for every wave of the block, so the block
    // barriers below are reached by all of its threads
    for (int64_t i0 = (int64_t)blockIdx.x * 4; i0 < p.count; i0 += stride) {
        const int64_t i = i0 + wv;
        const bool active = i < p.count;
        for (int w = lane; w < cw; w += 64) words[wv][w] = 0u;
        __syncthreads();
        float gg = 0.0f;
        if (active) {
            for (int c = lane; c < p.d; c += 64) {
                const float y = p.Y[i * p.d + c];
                uint32_t code = 0;
                float yh = lv[0];
                for (int k = 0; k < 15; ++k) {
                    const bool ge = y >= th[k];
                    code = ge ? (uint32_t)(k + 1) : code;
                    yh = ge ? lv[k + 1] : yh;
                }
                const float e = y - yh;
                p.U[i * p.d + c] = e;
                gg = fmaf(e, e, gg);
                const dev::CodeLoc L = dev::code_loc(c, p.bits);
                atomicOr(&words[wv][L.w0], (code & ((1u << L.n0) - 1u)) << L.s0);
                if (L.n0 < p.bits) atomicOr(&words[wv][L.w1], (code >> L.n0) << L.s1);
            }
        }
        gg = wave_sum(gg);
        __syncthreads();
        if (active) {
            int64_t off;
            int tok;
            const int64_t n = dense_record(p, p.start + i, &off, &tok);
            for (int w = lane; w < cw; w += 64) p.codes[n * cw + w] = words[wv][w];
            if (lane == 0 && p.m > 0) p.rnorm[n] = sqrtf(gg);
        }
        __syncthreads();
    }
}

// vector codebooks (FibQuant summary, section 2.3), one wave per vector: each
// block of `block` rotated coordinates of Y takes its nearest codeword - the
// largest <y, c> - |c|^2 / 2, ties to the smaller index - from the codebook
// in LDS; index j goes to bits [j bits, (j+1) bits) of the record, assembled
// in LDS
constexpr int kMaxVqWords = 4096 * 8 / 2 / 32;
__global__ __launch_bounds__(256) void dense_vq_kernel(DenseK p) {
    __shared__ uint32_t words[4][kMaxVqWords];
    __shared__ float s_code[256 * 4];  // {c_0 .. c_{k-1}, -|c|^2 / 2} per codeword
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int k = p.block, N = 1 << p.bits, nb = p.d / k;
    const int cw = (p.bits * nb + 31) / 32;
    for (int c = threadIdx.x; c < N; c += blockDim.x) {
        float h = 0.0f;
        for (int i = 0; i < k; ++i) {
            const float v = p.levels[c * k + i];
            s_code[4 * c + i] = v;
            h = fmaf(v, v, h);
        }
        s_code[4 * c + 3] = -0.5f * h;
    }
    const int64_t stride = (int64_t)gridDim.x * 4;
    // the loop bound is the same for every wave of the block, so the block
    // barriers below are reached by all of its threads
    for (int64_t i0 = (int64_t)blockIdx.x * 4; i0 < p.count; i0 += stride) {
        const int64_t i = i0 + wv;
        const bool active = i < p.count;
        for (int w = lane; w < cw; w += 64) words[wv][w] = 0u;
        __syncthreads();
        if (active) {
            for (int j = lane; j < nb; j += 64) {
                const float* y = p.Y + i * p.d + (int64_t)j * k;
                const float y0 = y[0], y1 = y[1], y2 = k == 3 ? y[2] : 0.0f;
                float bs = -INFINITY;
                uint32_t bi = 0;
                for (int c = 0; c < N; ++c) {
                    const float* cv = s_code + 4 * c;
                    float sc = fmaf(cv[1], y1, fmaf(cv[0], y0, cv[3]));
                    if (k == 3) sc = fmaf(cv[2], y2, sc);
                    if (sc > bs) {
                        bs = sc;
                        bi = (uint32_t)c;
                    }
                }
                const int o = j * p.bits;
                atomicOr(&words[wv][o >> 5], bi << (o & 31));
                if ((o & 31) + p.bits > 32) atomicOr(&words[wv][(o >> 5) + 1], bi >> (32 - (o & 31)));
            }
        }
        __syncthreads();
        if (active) {
            int64_t off;
            int tok;
            const int64_t n = dense_record(p, p.start + i, &off, &tok);
            for (int w = lane; w < cw; w += 64) p.codes[n * cw + w] = words[wv][w];
        }
        __syncthreads();
    }
}

// one wave per vector: sign bits of Z
__global__ __launch_bounds__(256) void dense_signs_kernel(DenseK p) {
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * 4;
    const int mw = p.m / 32;
    for (int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); i < p.count; i += stride) {
        int64_t off;
        int tok;
        const int64_t n = dense_record(p, p.start + i, &off, &tok);
        for (int c = 0; c < p.m; c += 64) {
            const int l = c + lane;
            const bool bit = l < p.m && p.Z[i * p.m + l] >= 0.0f;
            const uint64_t ball = __ballot(bit);
            if (lane == 0) p.signs[n * mw + c / 32] = (uint32_t)ball;
            if (lane == 32 && c / 32 + 1 < mw) p.signs[n * mw + c / 32 + 1] = (uint32_t)(ball >> 32);
        }
    }
}

int64_t dense_chunk(int64_t nvec) { return nvec < 65536 ? nvec : 65536; }

using EncFn = void (*)(EncK);

template <int D, int BITS, int M, int MODE, bool GEN>
EncFn pick_dtype_g(bool bf16, bool rope) {
    if (rope) return bf16 ? encode_had_kernel<D, BITS, M, true, true, MODE, GEN>
                          : encode_had_kernel<D, BITS, M, false, true, MODE, GEN>;
    return bf16 ? encode_had_kernel<D, BITS, M, true, false, MODE, GEN>
                : encode_had_kernel<D, BITS, M, false, false, MODE, GEN>;
}

// gen: the general-addressing kernel (appends, page tables)
template <int D, int BITS, int M, int MODE>
EncFn pick_dtype(bool bf16, bool rope, bool gen) {
    return gen ? pick_dtype_g<D, BITS, M, MODE, true>(bf16, rope) : pick_dtype_g<D, BITS, M, MODE, false>(bf16, rope);
}

template <int D, int BITS>
EncFn pick_m(int m, bool bf16, bool rope, int mode, bool gen) {
    if (mode != 0) {
        if constexpr (BITS <= 3) {
            if (m != D) return nullptr;
            return mode == 1 ? pick_dtype<D, BITS, D, 1>(bf16, rope, gen) : pick_dtype<D, BITS, D, 2>(bf16, rope, gen);
        }
        return nullptr;
    }
    if (m == 0) return pick_dtype<D, BITS, 0, 0>(bf16, rope, gen);
    if (m == D / 2) return pick_dtype<D, BITS, D / 2, 0>(bf16, rope, gen);
    if (m == D) return pick_dtype<D, BITS, D, 0>(bf16, rope, gen);
    return nullptr;
}

template <int D>
EncFn pick_bits(int bits, int m, bool bf16, bool rope, int mode, bool gen) {
    switch (bits) {
        case 1: return pick_m<D, 1>(m, bf16, rope, mode, gen);
        case 2: return pick_m<D, 2>(m, bf16, rope, mode, gen);
        case 3: return pick_m<D, 3>(m, bf16, rope, mode, gen);
        case 4: return pick_m<D, 4>(m, bf16, rope, mode, gen);
    }
    return nullptr;
}

template <int D>
EncFn pick_vq_bits(int bits, bool bf16, bool rope, bool gen) {
    switch (bits) {
        case 1: return pick_dtype<D, 1, 0, 3>(bf16, rope, gen);
        case 2: return pick_dtype<D, 2, 0, 3>(bf16, rope, gen);
        case 3: return pick_dtype<D, 3, 0, 3>(bf16, rope, gen);
        case 4: return pick_dtype<D, 4, 0, 3>(bf16, rope, gen);
        case 5: return pick_dtype<D, 5, 0, 3>(bf16, rope, gen);
        case 6: return pick_dtype<D, 6, 0, 3>(bf16, rope, gen);
        case 7: return pick_dtype<D, 7, 0, 3>(bf16, rope, gen);
        case 8: return pick_dtype<D, 8, 0, 3>(bf16, rope, gen);
    }
    return nullptr;
}

// mode: 0 QJL sketch, 1 sign correction, 2 sign correction without rotation,
// 3 vector codebook (bits = log2 of the codebook size)
EncFn pick_encode(int d, int bits, int m, bool bf16, bool rope, int mode, bool gen) {
    if (mode == 3) {
        if (d == 64) return pick_vq_bits<64>(bits, bf16, rope, gen);
        if (d == 128) return pick_vq_bits<128>(bits, bf16, rope, gen);
        return nullptr;
    }
    if (d == 64) return pick_bits<64>(bits, m, bf16, rope, mode, gen);
    if (d == 128) return pick_bits<128>(bits, m, bf16, rope, mode, gen);
    return nullptr;
}

int g_num_cus = 0;

// resident 256-thread blocks per CU of an encode kernel at a dynamic LDS size
int resident_per_cu(const void* fn, size_t lds) {
    static thread_local const void* last_fn = nullptr;
    static thread_local size_t last_lds = 0;
    static thread_local int last = 0;
    if (fn == last_fn && lds == last_lds) return last;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, lds) != hipSuccess || per_cu < 1) {
        (void)hipGetLastError();
        return 8;
    }
    last_fn = fn;
    last_lds = lds;
    last = per_cu;
    return per_cu;
}

}  // namespace

size_t encode_workspace_bytes(const tq_codebook* cb, int64_t n_vectors) {
    if (!cb->dense) return 0;
    const int64_t c = dense_chunk(n_vectors);
    return (size_t)c * (2 * (size_t)cb->spec.d + (size_t)cb->spec.m) * sizeof(float);
}

hipError_t launch_encode(const tq_codebook* cb, const EncodeArgs& a, hipStream_t stream) {
    const int d = cb->spec.d, bits = cb->spec.bits, m = cb->spec.m;
    if (!g_num_cus) {
        int dev = 0;
        hipDeviceProp_t prop;
        if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return hipErrorUnknown;
        g_num_cus = prop.multiProcessorCount;
    }
    if (cb->spec.block >= 2 && !vq_supported(cb)) return hipErrorInvalidValue;
    if (!cb->dense) {
        const int mode = cb->spec.block >= 2                    ? 3
                         : cb->spec.correction == TQ_CORR_SIGN ? (cb->spec.rotation == TQ_ROT_NONE ? 2 : 1)
                                                               : 0;
        // the bulk kernel stages RoPE rows per block of four heads; other head
        // counts take the general kernel (per-lane rows)
        const bool gen = a.append != 0 || a.pages.table != nullptr || (a.rope_cos != nullptr && a.h_kv % 4 != 0);
        EncFn fn = pick_encode(d, bits, m, a.bf16 != 0, a.rope_cos != nullptr, mode, gen);
        if (!fn) return hipErrorInvalidValue;
        EncK p{};
        p.x = a.x;
        p.s_seq = a.s_seq;
        p.s_tok = a.s_tok;
        p.s_head = a.s_head;
        p.n_seq = a.n_seq;
        p.n_tok = a.n_tok;
        p.h_kv = a.h_kv;
        p.tok_offset = a.tok_offset;
        p.L_cap = a.L_cap;
        p.tok_blocks = (a.n_tok + 31) / 32;
        p.n_tiles = (int64_t)a.n_seq * p.tok_blocks * a.h_kv;
        p.rope_cos = a.rope_cos;
        p.rope_sin = a.rope_sin;
        p.sigma = cb->dev.sigma;
        p.levels = cb->dev.levels;
        p.thresholds = cb->dev.thresholds;
        p.sketch_mfma = cb->dev.sketch_mfma;
        p.vq_grid = cb->dev.vq_grid;
        p.vq_inv_cell = cb->vq_inv_cell;
        p.norm = a.out.norm;
        p.rnorm = a.out.rnorm;
        p.codes = a.out.codes;
        p.signs = a.out.signs;
        p.rope_stage = (a.rope_cos != nullptr && a.h_kv % 4 == 0 && !a.append) ? 1 : 0;
        p.div_h = dev::FastDiv((uint32_t)a.h_kv);
        p.div_seq = dev::FastDiv((uint32_t)a.n_seq);
        p.append = a.append;
        p.pos = a.pos;
        p.rope_npos = a.rope_npos;
        p.pages = a.pages.table;
        p.page_size = a.pages.size;
        p.max_pages = a.pages.max_pages;
        p.n_pages = a.pages.n_pages;
        p.div_page = dev::FastDiv((uint32_t)(a.pages.size > 0 ? a.pages.size : 1));
        if (a.append) p.n_tiles = ((int64_t)a.n_seq * a.h_kv + 31) / 32;
        const size_t lds = p.rope_stage ? (size_t)2 * 32 * (d / 2 + 4) * sizeof(float) : 0;
        // persistent blocks: as many as are resident at once, so that no
        // partial last round of blocks leaves CUs idle
        const int64_t blocks_needed = (p.n_tiles + 3) / 4;
        const int64_t cap = (int64_t)g_num_cus * resident_per_cu((const void*)fn, lds);
        const int grid = (int)(blocks_needed < cap ? blocks_needed : cap);
        hipLaunchKernelGGL(fn, dim3(grid), dim3(256), lds, stream, p);
        return hipGetLastError();
    }
    // dense form, chunk by chunk
    const int64_t nvec = (int64_t)a.n_seq * a.n_tok * a.h_kv;
    const int64_t chunk = dense_chunk(nvec);
    float* U = static_cast<float*>(a.ws);
    float* Y = U + chunk * d;
    float* Z = Y + chunk * d;
    for (int64_t start = 0; start < nvec; start += chunk) {
        const int64_t cnt = (nvec - start) < chunk ? (nvec - start) : chunk;
        DenseK p{};
        p.x = a.x;
        p.s_seq = a.s_seq;
        p.s_tok = a.s_tok;
        p.s_head = a.s_head;
        p.n_tok = a.n_tok;
        p.h_kv = a.h_kv;
        p.tok_offset = a.tok_offset;
        p.L_cap = a.L_cap;
        p.d = d;
        p.m = m;
        p.bits = bits;
        p.block = cb->spec.block;
        p.start = start;
        p.count = cnt;
        p.bf16 = a.bf16;
        p.rope_cos = a.rope_cos;
        p.rope_sin = a.rope_sin;
        p.levels = cb->dev.levels;
        p.thresholds = cb->dev.thresholds;
        p.U = U;
        p.Y = Y;
        p.Z = Z;
        p.norm = a.out.norm;
        p.rnorm = a.out.rnorm;
        p.codes = a.out.codes;
        p.signs = a.out.signs;
        const int grid = (int)((cnt + 3) / 4 < (int64_t)g_num_cus * 8 ? (cnt + 3) / 4 : (int64_t)g_num_cus * 8);
        hipLaunchKernelGGL(dense_prep_kernel, dim3(grid), dim3(256), 0, stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_gemm_nt(U, d, cb->dev.rot, d, Y, d, (int)cnt, d, d, stream);
        if (e != hipSuccess) return e;
        if (cb->spec.block >= 2) hipLaunchKernelGGL(dense_vq_kernel, dim3(grid), dim3(256), 0, stream, p);
        else hipLaunchKernelGGL(dense_quant_kernel, dim3(grid), dim3(256), 0, stream, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (m > 0) {
            e = launch_gemm_nt(U, d, cb->dev.sketch, d, Z, m, (int)cnt, m, d, stream);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(dense_signs_kernel, dim3(grid), dim3(256), 0, stream, p);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace tq
