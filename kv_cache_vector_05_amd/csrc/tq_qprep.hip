// Query preparation for the integer-MFMA logit scan (tq_scan.hip) and the
// fused decode (tq_decode.hip) (tambur post: logits straight from quantised
// keys; iaemfoco post, "TurboQuant: Uma Nova Abordagem" and itstec post, "Por
// dentro do processo de compressao KV": the one-bit QJL correction):
//     q' = Pi RoPE(q),  s = S q'  (s = q' with the sign correction of the
//     TurboESM summary, technical section 2).
// Both are turned into fixed-point integers with one power-of-two scale per
// query (28 bits, |X| <= 2^26) and split into four balanced base-128 int8
// digits, the rows of the scan's and the decode's MFMA A operands; the scale
// and the exact sum of the fixed-point s values go beside them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

struct QDig {
    const void* q;
    int32_t bf16, Hq, L_cap, m, sdw, ncs;
    int64_t rows;     // B * Hq
    int32_t norot;    // Pi = I: q' = RoPE(q)
    int32_t s_ident;  // S = I (sign correction): s = q'
    const int32_t* seq_len;
    const int32_t* q_pos;
    const float* rope_cos;
    const float* rope_sin;
    const float* sigma;
    const float* sketch_t;  // S^T [D][m]
    int8_t* qd;      // [rows*4][D]  digits of q' (digit rows 4*row + a)
    int8_t* sd;      // [rows*4][sdw] digits of s in MFMA slot order
    float* scale;    // [rows][3]    shift(q'), shift(s), sum of the fixed-point s values
};

// One workgroup per query row (tq_device.h::Prep, the routine the scan runs
// in LDS for its own rows): the digits, scales and sums go to the workspace
// for the fused decode.
template <int D, int M>
__global__ __launch_bounds__(256) void qprep_digits_kernel(QDig p) {
    using PL = dev::PrepLds<D, M, 1>;
    __shared__ PL L;
    const int64_t row = blockIdx.x;
    const int b = (int)(row / p.Hq);
    dev::PrepIn in{};
    in.q = p.q;
    in.bf16 = p.bf16;
    in.L_cap = p.L_cap;
    in.norot = p.norot;
    in.s_ident = p.s_ident;
    in.rope_cos = p.rope_cos;
    in.rope_sin = p.rope_sin;
    in.sigma = p.sigma;
    in.sketch_t = p.sketch_t;
    dev::Prep<D, M, 1> pr;
    pr.load(in, [&](int) { return row; }, dev::query_pos(p.q_pos, p.seq_len, b, p.L_cap));
    pr.compute(in, L);
    const int t = threadIdx.x;
    const int8_t* qd = &L.qd[0][0][0];
    for (int i = t; i < 4 * D; i += 256) p.qd[row * 4 * D + i] = qd[i];
    if constexpr (M > 0) {
        const int8_t* sd = &L.sd[0][0][0];
        for (int i = t; i < 4 * PL::SDW; i += 256) p.sd[row * 4 * PL::SDW + i] = sd[i];
    }
    if (t < 3) p.scale[row * 3 + t] = L.scl[0][t];
}

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// the integer-digit tile of the fused decode serves the fused scan's codebooks
bool logits_mfma_supported(const tq_codebook* ck) { return scan_supported(ck); }

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
    p.rows = (int64_t)a.B * a.Hq;
    p.seq_len = a.seq_len;
    p.q_pos = a.q_pos;
    p.rope_cos = a.rope_cos;
    p.rope_sin = a.rope_sin;
    p.sigma = ck->dev.sigma;
    p.sketch_t = ck->dev.sketch_t;
    p.norot = no_rotation(ck) ? 1 : 0;
    p.s_ident = sign_corr(ck) ? 1 : 0;
    p.qd = q.qd;
    p.sd = q.sd;
    p.scale = q.scale;
    const unsigned grid = (unsigned)p.rows;
    if (grid == 0) return hipSuccess;
    using Fn = void (*)(QDig);
    Fn fn = nullptr;
    const bool d64 = ck->spec.d == 64;
    switch (p.m) {
        case 0: fn = d64 ? qprep_digits_kernel<64, 0> : qprep_digits_kernel<128, 0>; break;
        case 32: fn = d64 ? qprep_digits_kernel<64, 32> : qprep_digits_kernel<128, 32>; break;
        case 64: fn = d64 ? qprep_digits_kernel<64, 64> : qprep_digits_kernel<128, 64>; break;
        case 128: fn = d64 ? qprep_digits_kernel<64, 128> : qprep_digits_kernel<128, 128>; break;
    }
    if (!fn) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace tq
