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
// step's operands are loaded as fp32 through buffer resources over the tile's
// rows (float4 where rows are 16-byte aligned; columns past K read zeros),
// split while they are written to LDS (rows padded to 40 bf16, so that the
// 16-byte reads of an MFMA operand fall in distinct banks), and the operands
// of the step two ahead are loaded into registers while the current one
// multiplies.
#include <hip/hip_runtime.h>

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
constexpr int kLoads = kTile * kKt / 4 / 256;  // float4 slots per thread per operand and step
constexpr float kQjlF = 1.2533141373155003f;   // sqrt(pi / 2)

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
    constexpr uint32_t kOut = 0x80000000u;  // beyond any tile
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

// B rows from packed scalar records (the index scan): row n of B is key
// n0 + n's estimate in the rotated domain, t[c_i] for i < d and then
// sqrt(pi/2)/m gamma z_l (+-) for l < m; the same values a dequantisation
// pass would write (QJL estimator, iaemfoco post, "TurboQuant: Uma Nova
// Abordagem"), formed while the step is loaded.  d and m are multiples of
// 32, so a step lies in one part; BITS is 1, 2 or 4 (four codes in one
// word).  The resources span the tile's records: keys past the last read
// zeros, which only feed columns that are never stored.
struct RecTile {
    __amdgpu_buffer_rsrc_t codes, signs, rnorm;
    int cw, mw, d, m, K;
    float cq;
};
template <int BITS>
__device__ __forceinline__ void load_step_rec(const RecTile& R, const float* lv, int k0, int tid,
                                              float4 (&v)[kLoads]) {
    constexpr uint32_t mask = (1u << BITS) - 1u;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int idx = tid + 256 * i;
        const int kl = idx >> 3;
        const int k = k0 + 4 * (idx & 7);
        float x[4] = {0.f, 0.f, 0.f, 0.f};
        if (k0 < R.d) {  // the same for the whole workgroup
            const int bp = BITS * k;
            const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(R.codes, (uint32_t)(kl * R.cw + (bp >> 5)) * 4u, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = lv[(w >> ((bp & 31) + BITS * j)) & mask];
        } else if (k0 < R.K) {
            const int l = k - R.d;
            const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(R.signs, (uint32_t)(kl * R.mw + (l >> 5)) * 4u, 0, 0);
            const float g = R.cq * __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(R.rnorm, (uint32_t)kl * 4u, 0, 0));
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = ((w >> ((l + j) & 31)) & 1u) ? g : -g;
        }
        v[i] = make_float4(x[0], x[1], x[2], x[3]);
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
// L2 to the others (for the index scan, the dequantised keys against the
// few query tiles).
// BITS = 0: B is an fp32 matrix; 1, 2, 4: B is formed from packed records
template <bool VEC, int BITS>
__global__ __launch_bounds__(256) void gemm_nt_bf16x3(const float* __restrict__ A, int64_t lda,
                                                      const float* __restrict__ B, int64_t ldb,
                                                      float* __restrict__ C, int64_t ldc, int M, int N, int K,
                                                      int m_fast, RecB rec) {
    __shared__ __attribute__((aligned(16))) __bf16 As[3 * kPiece];
    __shared__ __attribute__((aligned(16))) __bf16 Bs[3 * kPiece];
    constexpr bool REC = BITS > 0;
    __shared__ float lvs[REC ? 16 : 1];  // record B: the level table
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int tm = (M + kTile - 1) / kTile, tn = (N + kTile - 1) / kTile;
    const int nf = m_fast ? tm : tn, ns = m_fast ? tn : tm;
    const int w = blockIdx.x, r = w >> 3;
    const int f = r % nf, sl = (r / nf) * 8 + (w & 7);
    if (sl >= ns) return;  // the last group's padding
    const int64_t m0 = (int64_t)(m_fast ? f : sl) * kTile;
    const int64_t n0 = (int64_t)(m_fast ? sl : f) * kTile;
    RecTile rt{};
    if constexpr (REC) {
        if (tid < (1 << BITS)) lvs[tid] = rec.levels[tid];
        rt.cw = BITS * rec.d / 32;
        rt.mw = rec.m / 32;
        rt.d = rec.d;
        rt.m = rec.m;
        rt.K = rec.d + rec.m;
        rt.cq = rec.m ? kQjlF / (float)rec.m : 0.f;
        const int64_t nk = N - n0 < kTile ? N - n0 : kTile, r0 = rec.rec0 + n0;
        rt.codes = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(rec.codes + r0 * rt.cw), (short)0,
                                                      (int)(nk * rt.cw * 4), 0x00020000);
        rt.signs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(rec.m ? rec.signs + r0 * rt.mw : nullptr),
                                                      (short)0, (int)(rec.m ? nk * rt.mw * 4 : 0), 0x00020000);
        rt.rnorm = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(rec.m ? rec.rnorm + r0 : nullptr), (short)0,
                                                      (int)(rec.m ? nk * 4 : 0), 0x00020000);
        __syncthreads();
    }
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
        if constexpr (REC) load_step_rec<BITS>(rt, lvs, s * kKt, tid, vb[s]);
        else load_step<VEC>(rb, ldb, s * kKt, K, tid, vb[s]);
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
            if constexpr (REC) load_step_rec<BITS>(rt, lvs, k0 + (h + 2) * kKt, tid, vb[h]);
            else load_step<VEC>(rb, ldb, k0 + (h + 2) * kKt, K, tid, vb[h]);
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
    // D[i][j] of a 32x32 block: column j = lane % 32, row 8*(r/4) + 4*(lane/32) + r%4
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

}  // namespace

namespace {
template <int BITS>
void launch_kernel(bool vec, dim3 grid, hipStream_t stream, const float* A, int64_t lda, const float* B, int64_t ldb,
                   float* C, int64_t ldc, int M, int N, int K, int m_fast, const RecB& r) {
    if (vec) hipLaunchKernelGGL((gemm_nt_bf16x3<true, BITS>), grid, dim3(256), 0, stream, A, lda, B, ldb, C, ldc, M, N, K, m_fast, r);
    else hipLaunchKernelGGL((gemm_nt_bf16x3<false, BITS>), grid, dim3(256), 0, stream, A, lda, B, ldb, C, ldc, M, N, K, m_fast, r);
}

hipError_t launch_gemm(const float* A, int64_t lda, const float* B, int64_t ldb, const RecB* rec, float* C,
                       int64_t ldc, int M, int N, int K, hipStream_t stream) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const int64_t tm = (M + kTile - 1) / kTile, tn = (N + kTile - 1) / kTile;
    const int m_fast = tm <= tn ? 1 : 0;
    const int64_t nf = m_fast ? tm : tn, ns = m_fast ? tn : tm;
    const int64_t blocks = nf * ((ns + 7) / 8) * 8;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    // float4 loads need 16-byte aligned rows
    const bool vec = ((lda | (rec ? 0 : ldb)) & 3) == 0 &&
                     ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(rec ? nullptr : B)) & 15) == 0;
    const RecB r = rec ? *rec : RecB{};
    const dim3 grid((unsigned)blocks);
    switch (rec ? rec->bits : 0) {
        case 0: launch_kernel<0>(vec, grid, stream, A, lda, B, ldb, C, ldc, M, N, K, m_fast, r); break;
        case 1: launch_kernel<1>(vec, grid, stream, A, lda, B, ldb, C, ldc, M, N, K, m_fast, r); break;
        case 2: launch_kernel<2>(vec, grid, stream, A, lda, B, ldb, C, ldc, M, N, K, m_fast, r); break;
        case 4: launch_kernel<4>(vec, grid, stream, A, lda, B, ldb, C, ldc, M, N, K, m_fast, r); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_nt(const float* A, int64_t lda, const float* B, int64_t ldb, float* C,
                          int64_t ldc, int M, int N, int K, hipStream_t stream) {
    return launch_gemm(A, lda, B, ldb, nullptr, C, ldc, M, N, K, stream);
}

hipError_t launch_gemm_records(const float* A, int64_t lda, const RecB& rec, float* C, int64_t ldc, int M, int N,
                               hipStream_t stream) {
    if (rec.d % 32 != 0 || rec.m % 32 != 0 || !(rec.bits == 1 || rec.bits == 2 || rec.bits == 4))
        return hipErrorInvalidValue;
    return launch_gemm(A, lda, nullptr, 0, &rec, C, ldc, M, N, rec.d + rec.m, stream);
}

}  // namespace tq
