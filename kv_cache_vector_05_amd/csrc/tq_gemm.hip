// Plain fp32 GEMM on CDNA MFMA: C[M][N] = A[M][K] * B[N][K]^T, row-major
// operands with the K index contiguous.  Used by the dense (Haar) rotation
// path: rotating unit vectors by Pi, sketching residuals by S, preparing
// queries, and scoring a dense-rotation index.
//
// Tiling: 256 threads (4 wave64s) own a 128 x 128 tile of C; each wave owns a
// 64 x 64 quarter as 2 x 2 blocks of v_mfma_f32_32x32x2f32.  K advances in
// steps of 32 through LDS tiles padded to 33 floats per row so that the 32
// rows an MFMA operand reads fall in distinct banks.  The next step's operands
// are loaded into registers (float4 where rows are 16-byte aligned) while the
// current step multiplies, so global latency overlaps the matrix work.
#include <hip/hip_runtime.h>

#include "tq_internal.h"

namespace tq {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 128;
constexpr int kKt = 32;
constexpr int kLd = kKt + 1;
constexpr int kLoads = kTile * kKt / 4 / 256;  // float4 slots per thread per operand and step

// rows m0 + idx/8 of X, columns k0 + 4 (idx % 8) .. + 3 for the thread's slots
template <bool VEC>
__device__ __forceinline__ void load_step(const float* __restrict__ X, int64_t ldx, int64_t r0, int rows, int k0,
                                          int K, int tid, float4 (&v)[kLoads]) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int idx = tid + 256 * i;
        const int64_t r = r0 + (idx >> 3);
        const int k = k0 + 4 * (idx & 7);
        if constexpr (VEC) {
            v[i] = (r < rows && k < K) ? *reinterpret_cast<const float4*>(X + r * ldx + k) : make_float4(0.f, 0.f, 0.f, 0.f);
        } else {
            const bool ok = r < rows;
            v[i].x = ok && k < K ? X[r * ldx + k] : 0.f;
            v[i].y = ok && k + 1 < K ? X[r * ldx + k + 1] : 0.f;
            v[i].z = ok && k + 2 < K ? X[r * ldx + k + 2] : 0.f;
            v[i].w = ok && k + 3 < K ? X[r * ldx + k + 3] : 0.f;
        }
    }
}

__device__ __forceinline__ void store_step(float* S, int tid, const float4 (&v)[kLoads]) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int idx = tid + 256 * i;
        float* d = S + (idx >> 3) * kLd + 4 * (idx & 7);
        d[0] = v[i].x;
        d[1] = v[i].y;
        d[2] = v[i].z;
        d[3] = v[i].w;
    }
}

template <bool VEC>
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

    float4 va[kLoads], vb[kLoads];
    load_step<VEC>(A, lda, m0, M, 0, K, tid, va);
    load_step<VEC>(B, ldb, n0, N, 0, K, tid, vb);
    for (int k0 = 0; k0 < K; k0 += kKt) {
        store_step(As, tid, va);
        store_step(Bs, tid, vb);
        __syncthreads();
        if (k0 + kKt < K) {  // the next step's operands, in flight during this step
            load_step<VEC>(A, lda, m0, M, k0 + kKt, K, tid, va);
            load_step<VEC>(B, ldb, n0, N, k0 + kKt, K, tid, vb);
        }
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
    // float4 loads need 16-byte aligned rows
    const bool vec = ((lda | ldb) & 3) == 0 && ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) & 15) == 0;
    if (vec) hipLaunchKernelGGL(gemm_nt_f32<true>, grid, dim3(256), 0, stream, A, lda, B, ldb, C, ldc, M, N, K);
    else hipLaunchKernelGGL(gemm_nt_f32<false>, grid, dim3(256), 0, stream, A, lda, B, ldb, C, ldc, M, N, K);
    return hipGetLastError();
}

}  // namespace tq
