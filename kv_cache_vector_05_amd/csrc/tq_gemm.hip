// fp32 GEMM on the bf16 matrix cores: C[M][N] = A[M][K] * B[N][K]^T,
// row-major operands with the K index contiguous.  Used by the dense (Haar)
// rotation path: rotating unit vectors by Pi, sketching residuals by S,
// preparing queries, and scoring a dense-rotation index.
//
// Each fp32 operand is split into three bf16 pieces, x = h + m + l (each the
// remainder of the previous, rounded to nearest: |x - h - m - l| <= 2^-27 |x|
// with bf16's 8-bit significands and fp32's exponent range, so no scaling is
// needed).  A product keeps the six piece products down to the 2^-16 level,
//     a b ~ ah bh + ah bm + am bh + ah bl + al bh + am bm,
// and leaves out am bl, al bm, al bl (each below 2^-24 |a b|, the rounding of
// an fp32 product).  Six v_mfma_f32_32x32x16_bf16 per 16 K-steps against the
// 64 K-steps of eight v_mfma_f32_32x32x2_f32: about 2.7 times the fp32
// matrix rate, with fp32 accumulation as before.
//
// Tiling: 256 threads (4 wave64s) own a 128 x 128 tile of C; each wave owns a
// 64 x 64 quarter as 2 x 2 blocks of 32 x 32.  K advances in steps of 32: the
// step's operands are loaded through buffer resources over the tile's rows
// (columns past K read zeros), written to LDS as three piece planes (rows
// padded to 40 bf16, so that the 16-byte reads of an MFMA operand fall in
// distinct banks), and the operands of the step two ahead are loaded into
// registers while the current one multiplies.
//
// The index scan has a kernel of its own (gemm_rec_kernel): its queries
// arrive split once into piece planes, and its keys are formed from their
// packed records while they are loaded.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 128;
constexpr int kKt = 32;
constexpr int kRow = kKt + 8;                  // bf16 per LDS row
constexpr int kPiece = kTile * kRow;           // bf16 per piece plane
constexpr int kLoads = kTile * kKt / 4 / 256;  // four-element slots per thread per operand and step
constexpr float kQjlF = 1.2533141373155003f;   // sqrt(pi / 2)
constexpr uint32_t kOut = 0x80000000u;         // a buffer offset beyond any tile: reads zeros

// buffer resource over the tile's rows [r0, r0 + 128) of X (fewer at the
// last tile); loads past it return zeros
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const float* X, int64_t ldx, int64_t r0, int rows) {
    const int64_t n = rows - r0 < kTile ? rows - r0 : kTile;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(X + r0 * ldx), (short)0, (int)(n * ldx * 4), 0x00020000);
}

// rows idx/8 of the tile, columns k0 + 4 (idx % 8) .. + 3 for the thread's
// slots.  Every load is issued (columns past K read at an offset past the
// tile, which returns zeros), so no load sits behind a branch and the waits
// for one step leave the next step's loads in flight.
template <bool VEC>
__device__ __forceinline__ void load_step(__amdgpu_buffer_rsrc_t X, int64_t ldx, int k0, int K, int tid,
                                          float4 (&v)[kLoads]) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int idx = tid + 256 * i;
        const int k = k0 + 4 * (idx & 7);
        const uint32_t o = (uint32_t)(((idx >> 3) * ldx + k) * 4);
        if constexpr (VEC) {
            v[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(X, k < K ? o : kOut, 0, 0));
        } else {
            v[i].x = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(X, k < K ? o : kOut, 0, 0));
            v[i].y = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(X, k + 1 < K ? o + 4 : kOut, 0, 0));
            v[i].z = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(X, k + 2 < K ? o + 8 : kOut, 0, 0));
            v[i].w = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(X, k + 3 < K ? o + 12 : kOut, 0, 0));
        }
    }
}

// the three bf16 pieces of a pair of floats, packed two to a word
__device__ __forceinline__ void split3(float a, float b, uint32_t& h, uint32_t& m, uint32_t& l) {
    h = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});
    const float ra = a - __uint_as_float(h << 16), rb = b - __uint_as_float(h & 0xFFFF0000u);
    m = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)ra, (__bf16)rb});
    const float sa = ra - __uint_as_float(m << 16), sb = rb - __uint_as_float(m & 0xFFFF0000u);
    l = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)sa, (__bf16)sb});
}

// the thread's slots split into the three piece planes of S
__device__ __forceinline__ void store_step(__bf16* S, int tid, const float4 (&v)[kLoads]) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int idx = tid + 256 * i;
        const int o = (idx >> 3) * kRow + 4 * (idx & 7);
        uint32_t h0, m0, l0, h1, m1, l1;
        split3(v[i].x, v[i].y, h0, m0, l0);
        split3(v[i].z, v[i].w, h1, m1, l1);
        *reinterpret_cast<u32x2*>(S + o) = u32x2{h0, h1};
        *reinterpret_cast<u32x2*>(S + kPiece + o) = u32x2{m0, m1};
        *reinterpret_cast<u32x2*>(S + 2 * kPiece + o) = u32x2{l0, l1};
    }
}

// MFMA operand: row `row` of the tile, K slots 8 (lane / 32) .. + 7 of the
// 16-wide sub-step kk, from piece plane p
__device__ __forceinline__ bf16x8 operand(const __bf16* S, int p, int row, int kk, int lane) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(S + p * kPiece + row * kRow + 16 * kk + 8 * (lane >> 5)));
}

// Tile order: workgroup w of a one-dimensional grid takes tile (f, s) of a
// "fast" axis with nf tiles (the one with fewer) and a "slow" axis, as
// w = s % 8 + 8 (f + nf (s / 8)).  Workgroups are dealt to the eight XCDs in
// turn, so every tile sharing the slow index s runs on one XCD, together:
// that operand's 128 rows are read from HBM once and served from that XCD's
// L2 to the others (for the index scan, the keys against the few query
// tiles).  Returns false for the last group's padding.
__device__ __forceinline__ bool tile_of(int M, int N, int m_fast, int64_t& m0, int64_t& n0) {
    const int tm = (M + kTile - 1) / kTile, tn = (N + kTile - 1) / kTile;
    const int nf = m_fast ? tm : tn, ns = m_fast ? tn : tm;
    const int w = blockIdx.x, r = w >> 3;
    const int f = r % nf, sl = (r / nf) * 8 + (w & 7);
    if (sl >= ns) return false;
    m0 = (int64_t)(m_fast ? f : sl) * kTile;
    n0 = (int64_t)(m_fast ? sl : f) * kTile;
    return true;
}

// D[i][j] of a 32x32 block: column j = lane % 32, row 8*(r/4) + 4*(lane/32) + r%4
__device__ __forceinline__ void store_c(float* C, int64_t ldc, int M, int N, int64_t m0, int64_t n0, int wm, int wn,
                                        int lane, const floatx16 (&acc)[2][2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn + 32 * j + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row < M && col < N) C[row * ldc + col] = acc[i][j][r];
            }
        }
}

template <bool VEC>
__global__ __launch_bounds__(256) void gemm_nt_bf16x3(const float* __restrict__ A, int64_t lda,
                                                      const float* __restrict__ B, int64_t ldb,
                                                      float* __restrict__ C, int64_t ldc, int M, int N, int K,
                                                      int m_fast) {
    __shared__ __attribute__((aligned(16))) __bf16 As[3 * kPiece];
    __shared__ __attribute__((aligned(16))) __bf16 Bs[3 * kPiece];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int64_t m0, n0;
    if (!tile_of(M, N, m_fast, m0, n0)) return;
    const int wm = (wave >> 1) * 64;  // wave's row offset inside the tile
    const int wn = (wave & 1) * 64;

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // operands of two steps in flight: step s + 2 is requested once step s
    // is in LDS, so each load has two steps of matrix work to arrive in
    const __amdgpu_buffer_rsrc_t ra = tile_rsrc(A, lda, m0, M), rb = tile_rsrc(B, ldb, n0, N);
    float4 va[2][kLoads], vb[2][kLoads];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        load_step<VEC>(ra, lda, s * kKt, K, tid, va[s]);
        load_step<VEC>(rb, ldb, s * kKt, K, tid, vb[s]);
    }
    // K-steps in pairs, one per register buffer: the buffered operands split
    // into LDS, the step two ahead requested into the same registers, then
    // the step's MFMAs.  Steps past K (at most one, when their count is odd,
    // and the requests ahead) read zeros and add nothing.
    for (int k0 = 0; k0 < K; k0 += 2 * kKt) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            store_step(As, tid, va[h]);
            store_step(Bs, tid, vb[h]);
            __syncthreads();
            load_step<VEC>(ra, lda, k0 + (h + 2) * kKt, K, tid, va[h]);
            load_step<VEC>(rb, ldb, k0 + (h + 2) * kKt, K, tid, vb[h]);
#pragma unroll
            for (int kk = 0; kk < kKt / 16; ++kk) {
                bf16x8 a[2][3], b[2][3];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int p = 0; p < 3; ++p) {
                        a[i][p] = operand(As, p, wm + 32 * i + (lane & 31), kk, lane);
                        b[i][p] = operand(Bs, p, wn + 32 * i + (lane & 31), kk, lane);
                    }
                // smallest terms first: each enters the fp32 sum before the larger ones
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        floatx16 c = acc[i][j];
                        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][1], b[j][1], c, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][0], b[j][2], c, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][2], b[j][0], c, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][0], b[j][1], c, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][1], b[j][0], c, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][0], b[j][0], c, 0, 0, 0);
                        acc[i][j] = c;
                    }
            }
            __syncthreads();
        }
    }
    store_c(C, ldc, M, N, m0, n0, wm, wn, lane, acc);
}

// ---------------------------------------------------------------- index scan
// Rows of A split once into three bf16 piece planes [3][M][K]
__global__ __launch_bounds__(256) void split_rows_kernel(const float* __restrict__ A, int64_t lda, int M, int K,
                                                         __bf16* __restrict__ P) {
    const int64_t plane = (int64_t)M * K;
    const int64_t pairs = plane / 2;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < pairs; e += (int64_t)gridDim.x * 256) {
        const int64_t i = 2 * e, r = i / K;
        const int k = (int)(i - r * K);  // K is even: a pair lies in one row
        uint32_t h, m, l;
        split3(A[r * lda + k], A[r * lda + k + 1], h, m, l);
        reinterpret_cast<uint32_t*>(P)[e] = h;
        reinterpret_cast<uint32_t*>(P + plane)[e] = m;
        reinterpret_cast<uint32_t*>(P + 2 * plane)[e] = l;
    }
}

// Scores C[M][N] = A B^T of the queries' A = [q' | s] (split once into piece
// planes, K = d + m) against B = key n0 + n's rotated-domain estimate, formed
// from its packed record (QJL estimator, iaemfoco post, "TurboQuant: Uma
// Nova Abordagem"): t[c_i] for i < d, then sqrt(pi/2)/m gamma z_l, z = +-1.
//   * The sketch part runs first.  Its B is +-1, one exact bf16 piece, so a
//     step takes three products (a_l, a_m, a_h against it) instead of six;
//     then each accumulator column is multiplied once by its key's
//     sqrt(pi/2)/m gamma (fp32, one rounding).
//   * The level part adds t[c] on top, its three pieces read from a table of
//     the 2^BITS levels (BITS = 1, 2, 4: four codes in one word).
// d and m are multiples of 32, so a K-step lies in one part.  The resources
// span the tile's records: keys past the last read zeros and only feed
// columns that are never stored.
template <int BITS>
__global__ __launch_bounds__(256) void gemm_rec_kernel(const __bf16* __restrict__ Ap, int64_t plane, int M,
                                                       float* __restrict__ C, int64_t ldc, int N, int m_fast, RecB rec) {
    __shared__ __attribute__((aligned(16))) __bf16 As[3 * kPiece];
    __shared__ __attribute__((aligned(16))) __bf16 Bs[3 * kPiece];
    __shared__ uint16_t lvp[3][16];  // the levels' bf16 pieces
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int64_t m0, n0;
    if (!tile_of(M, N, m_fast, m0, n0)) return;
    const int wm = (wave >> 1) * 64;
    const int wn = (wave & 1) * 64;
    const int d = rec.d, m = rec.m, K = d + m;
    const int cw = BITS * d / 32, mw = m / 32;
    if (tid < 16) {
        uint32_t h, mm, l;
        split3(tid < (1 << BITS) ? rec.levels[tid] : 0.f, 0.f, h, mm, l);
        lvp[0][tid] = (uint16_t)h;
        lvp[1][tid] = (uint16_t)mm;
        lvp[2][tid] = (uint16_t)l;
    }
    // A planes over the tile's rows (piece p at a scalar offset of `plane`
    // elements); records of the tile's keys
    const int64_t mrows = M - m0 < kTile ? M - m0 : kTile;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16*>(Ap + m0 * K), (short)0, (int)((2 * plane + mrows * K) * 2), 0x00020000);
    const int64_t nk = N - n0 < kTile ? N - n0 : kTile, r0 = rec.rec0 + n0;
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(rec.codes + r0 * cw), (short)0, (int)(nk * cw * 4), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(m ? rec.signs + r0 * mw : nullptr), (short)0, (int)(m ? nk * mw * 4 : 0), 0x00020000);
    const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(m ? rec.rnorm + r0 : nullptr), (short)0, (int)(m ? nk * 4 : 0), 0x00020000);
    __syncthreads();

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // one K-step's raw operands: the A pieces of the thread's slots and one
    // record word per slot (codes or sign bits)
    struct Raw {
        u32x2 a[kLoads][3];
        uint32_t w[kLoads];
    };
    // step k0 of a part ending at ke (past ke: zeros)
    auto load = [&](int k0, int ke, bool sign, Raw& x) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int idx = tid + 256 * i;
            const int row = idx >> 3;  // A row, and B key, of the slot
            const int k = k0 + 4 * (idx & 7);
            const uint32_t oa = k0 < ke ? (uint32_t)((row * K + k) * 2) : kOut;
#pragma unroll
            for (int p = 0; p < 3; ++p)
                x.a[i][p] = __builtin_amdgcn_raw_buffer_load_b64(ra, oa, (uint32_t)(p * plane * 2), 0);
            uint32_t ob;
            if (sign) ob = k0 < ke ? (uint32_t)((row * mw + ((k - d) >> 5)) * 4) : kOut;
            else ob = k0 < ke ? (uint32_t)((row * cw + ((BITS * k) >> 5)) * 4) : kOut;
            x.w[i] = __builtin_amdgcn_raw_buffer_load_b32(sign ? rs : rc, ob, 0, 0);
        }
    };
    // the step's operands into LDS; a sign step writes B's first plane only
    auto store = [&](int k0, bool sign, const Raw& x) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int idx = tid + 256 * i;
            const int o = (idx >> 3) * kRow + 4 * (idx & 7);
            const int k = k0 + 4 * (idx & 7);
#pragma unroll
            for (int p = 0; p < 3; ++p) *reinterpret_cast<u32x2*>(As + p * kPiece + o) = x.a[i][p];
            if (sign) {
                // bit set: +1 (bf16 0x3F80), clear: -1 (0xBF80)
                const uint32_t b = x.w[i] >> ((k - d) & 31);
                const uint32_t lo = 0xBF80BF80u ^ (((b & 1u) << 15) | ((b & 2u) << 30));
                const uint32_t hi = 0xBF80BF80u ^ ((((b >> 2) & 1u) << 15) | (((b >> 2) & 2u) << 30));
                *reinterpret_cast<u32x2*>(Bs + o) = u32x2{lo, hi};
            } else {
                constexpr uint32_t mask = (1u << BITS) - 1u;
                const uint32_t b = x.w[i] >> ((BITS * k) & 31);
                const uint32_t c0 = b & mask, c1 = (b >> BITS) & mask, c2 = (b >> (2 * BITS)) & mask,
                               c3 = (b >> (3 * BITS)) & mask;
#pragma unroll
                for (int p = 0; p < 3; ++p)
                    *reinterpret_cast<u32x2*>(Bs + p * kPiece + o) =
                        u32x2{(uint32_t)lvp[p][c0] | ((uint32_t)lvp[p][c1] << 16),
                              (uint32_t)lvp[p][c2] | ((uint32_t)lvp[p][c3] << 16)};
            }
        }
    };
    // the steps of part [kb, ke) in pairs, two steps of loads in flight
    // (steps past ke, at most one when their count is odd, add zeros)
    auto part = [&](int kb, int ke, bool sign) {
        Raw x[2];
        load(kb, ke, sign, x[0]);
        load(kb + kKt, ke, sign, x[1]);
        for (int k0 = kb; k0 < ke; k0 += 2 * kKt) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                store(k0 + h * kKt, sign, x[h]);
                __syncthreads();
                load(k0 + (h + 2) * kKt, ke, sign, x[h]);
#pragma unroll
                for (int kk = 0; kk < kKt / 16; ++kk) {
                    bf16x8 a[2][3], b[2][3];
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int p = 0; p < 3; ++p) {
                            a[i][p] = operand(As, p, wm + 32 * i + (lane & 31), kk, lane);
                            b[i][p] = operand(Bs, sign ? 0 : p, wn + 32 * i + (lane & 31), kk, lane);
                        }
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            floatx16 c = acc[i][j];
                            if (sign) {
                                c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][2], b[j][0], c, 0, 0, 0);
                                c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][1], b[j][0], c, 0, 0, 0);
                            } else {
                                c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][1], b[j][1], c, 0, 0, 0);
                                c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][0], b[j][2], c, 0, 0, 0);
                                c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][2], b[j][0], c, 0, 0, 0);
                                c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][0], b[j][1], c, 0, 0, 0);
                                c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][1], b[j][0], c, 0, 0, 0);
                            }
                            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][0], b[j][0], c, 0, 0, 0);
                            acc[i][j] = c;
                        }
                }
                __syncthreads();
            }
        }
    };
    if (m > 0) {
        part(d, K, true);
        // each column's common factor sqrt(pi/2)/m gamma, once
        const float cq = kQjlF / (float)m;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int kl = wn + 32 * j + (lane & 31);
            const float g = cq * __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, (uint32_t)kl * 4u, 0, 0));
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] *= g;
        }
    }
    part(0, d, false);
    store_c(C, ldc, M, N, m0, n0, wm, wn, lane, acc);
}

// the one-dimensional XCD-grouped grid of an M x N output
struct Grid {
    dim3 grid;
    int m_fast;
    bool ok;
};
Grid grid_of(int M, int N) {
    const int64_t tm = (M + kTile - 1) / kTile, tn = (N + kTile - 1) / kTile;
    const int m_fast = tm <= tn ? 1 : 0;
    const int64_t nf = m_fast ? tm : tn, ns = m_fast ? tn : tm;
    const int64_t blocks = nf * ((ns + 7) / 8) * 8;
    return Grid{dim3((unsigned)blocks), m_fast, blocks <= 0x7FFFFFFF};
}

}  // namespace

hipError_t launch_gemm_nt(const float* A, int64_t lda, const float* B, int64_t ldb, float* C,
                          int64_t ldc, int M, int N, int K, hipStream_t stream) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const Grid g = grid_of(M, N);
    if (!g.ok) return hipErrorInvalidValue;
    // float4 loads need 16-byte aligned rows
    const bool vec = ((lda | ldb) & 3) == 0 && ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) & 15) == 0;
    if (vec) hipLaunchKernelGGL(gemm_nt_bf16x3<true>, g.grid, dim3(256), 0, stream, A, lda, B, ldb, C, ldc, M, N, K, g.m_fast);
    else hipLaunchKernelGGL(gemm_nt_bf16x3<false>, g.grid, dim3(256), 0, stream, A, lda, B, ldb, C, ldc, M, N, K, g.m_fast);
    return hipGetLastError();
}

bool gemm_records_supported(int d, int m, int bits) {
    return d > 0 && d % 32 == 0 && m % 32 == 0 && (bits == 1 || bits == 2 || bits == 4);
}

size_t gemm_records_split_bytes(int64_t M, int d, int m) { return (size_t)(3 * M * (d + m) * 2); }

hipError_t launch_split_rows(const float* A, int64_t lda, int M, int K, void* planes, hipStream_t stream) {
    if (M <= 0 || K <= 0) return hipSuccess;
    if (K % 2) return hipErrorInvalidValue;
    const int64_t pairs = (int64_t)M * K / 2;
    const unsigned blocks = (unsigned)std::min<int64_t>((pairs + 255) / 256, 65536);
    hipLaunchKernelGGL(split_rows_kernel, dim3(blocks), dim3(256), 0, stream, A, lda, M, K,
                       static_cast<__bf16*>(planes));
    return hipGetLastError();
}

hipError_t launch_gemm_records(const void* planes, int64_t plane, int M, const RecB& rec, float* C, int64_t ldc,
                               int N, hipStream_t stream) {
    if (!gemm_records_supported(rec.d, rec.m, rec.bits)) return hipErrorInvalidValue;
    if (M <= 0 || N <= 0) return hipSuccess;
    const Grid g = grid_of(M, N);
    if (!g.ok) return hipErrorInvalidValue;
    const __bf16* P = static_cast<const __bf16*>(planes);
    switch (rec.bits) {
        case 1: hipLaunchKernelGGL(gemm_rec_kernel<1>, g.grid, dim3(256), 0, stream, P, plane, M, C, ldc, N, g.m_fast, rec); break;
        case 2: hipLaunchKernelGGL(gemm_rec_kernel<2>, g.grid, dim3(256), 0, stream, P, plane, M, C, ldc, N, g.m_fast, rec); break;
        case 4: hipLaunchKernelGGL(gemm_rec_kernel<4>, g.grid, dim3(256), 0, stream, P, plane, M, C, ldc, N, g.m_fast, rec); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tq
