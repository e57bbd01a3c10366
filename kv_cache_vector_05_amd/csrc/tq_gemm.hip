// Plain fp32 GEMM on CDNA MFMA: C[M][N] = A[M][K] * B[N][K]^T, row-major
// operands with the K index contiguous.  Used by the dense (Haar) rotation
// path: rotating unit vectors by Pi, sketching residuals by S, preparing
// queries, and scoring a dense-rotation index.
//
// Tiling: 256 threads (4 wave64s) own a 128 x 128 tile of C; each wave owns a
// 64 x 64 quarter as 2 x 2 blocks of v_mfma_f32_32x32x2f32.  K advances in
// steps of 16 through LDS tiles padded to 17 floats per row so that the 32
// rows an MFMA operand reads fall in distinct banks.
#include <hip/hip_runtime.h>

#include "tq_internal.h"

namespace tq {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 128;
constexpr int kKt = 16;
constexpr int kLd = kKt + 1;

__global__ __launch_bounds__(256) void gemm_nt_f32(const float* __restrict__ A, int64_t lda,
                                                   const float* __restrict__ B, int64_t ldb,
                                                   float* __restrict__ C, int64_t ldc, int M, int N,
                                                   int K) {
    __shared__ float As[kTile * kLd];
    __shared__ float Bs[kTile * kLd];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * kTile;
    const int64_t n0 = (int64_t)blockIdx.x * kTile;
    const int wm = (wave >> 1) * 64;  // wave's row offset inside the tile
    const int wn = (wave & 1) * 64;

    floatx16 acc[2][2];
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j)
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // each thread stages 8 floats of A and 8 of B per K step:
    // rows (tid >> 2) and (tid >> 2) + 64, columns (tid & 3) * 4 .. + 3
    const int lr = tid >> 2;
    const int lc = (tid & 3) * 4;
    for (int k0 = 0; k0 < K; k0 += kKt) {
        for (int h = 0; h < 2; ++h) {
            const int row = lr + 64 * h;
            const int64_t ga = m0 + row, gb = n0 + row;
            for (int c = 0; c < 4; ++c) {
                const int kk = k0 + lc + c;
                As[row * kLd + lc + c] = (ga < M && kk < K) ? A[ga * lda + kk] : 0.0f;
                Bs[row * kLd + lc + c] = (gb < N && kk < K) ? B[gb * ldb + kk] : 0.0f;
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kKt; kk += 2) {
            const int kidx = kk + (lane >> 5);
            float a[2], b[2];
            for (int i = 0; i < 2; ++i) a[i] = As[(wm + 32 * i + (lane & 31)) * kLd + kidx];
            for (int j = 0; j < 2; ++j) b[j] = Bs[(wn + 32 * j + (lane & 31)) * kLd + kidx];
            for (int i = 0; i < 2; ++i)
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
    // D[i][j] of a 32x32 block: column j = lane % 32, row 8*(r/4) + 4*(lane/32) + r%4
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn + 32 * j + (lane & 31);
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row < M && col < N) C[row * ldc + col] = acc[i][j][r];
            }
        }
}

}  // namespace

hipError_t launch_gemm_nt(const float* A, int64_t lda, const float* B, int64_t ldb, float* C,
                          int64_t ldc, int M, int N, int K, hipStream_t stream) {
    if (M <= 0 || N <= 0) return hipSuccess;
    dim3 grid((N + kTile - 1) / kTile, (M + kTile - 1) / kTile);
    hipLaunchKernelGGL(gemm_nt_f32, grid, dim3(256), 0, stream, A, lda, B, ldb, C, ldc, M, N, K);
    return hipGetLastError();
}

}  // namespace tq
