// Internal declarations shared by the host side of libtq (argument checks,
// table construction, launch orchestration) and the HIP kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/tq.h"

namespace tq {

constexpr int kMaxLevels = 16;  // 2^bits for bits <= 4

struct DeviceTables {
    float* levels = nullptr;      // [16]   float32 Lloyd-Max levels (first K used)
    float* thresholds = nullptr;  // [16]   float32 thresholds (first K-1 used)
    float* sigma = nullptr;       // [d]    Hadamard signs as +-1.0f
    float* rot = nullptr;         // [d*d]  dense Pi, row-major (y = Pi u)
    float* sketch = nullptr;      // [m*d]  S, row-major
    float* sketch_mfma = nullptr; // [m*d]  S as fp16 hi/lo pairs in the encode kernel's MFMA operand order
    float* sketch_t = nullptr;    // [d*m]  S transposed (column l of S^T is row l of S)
    float* mu = nullptr;          // [n_mu] mean residual magnitudes (sign correction)
    uint32_t* vq_grid = nullptr;  // [kVqGrid^2] candidate codewords per cell (vector codebooks, N <= 64)
};

// Candidate grid of a two-coordinate vector codebook: kVqGrid^2 cells of side
// 1 / inv_cell over |y_i| < kVqGrid / (2 inv_cell); cell (ix, iy) holds, in
// bytes 0..3 of word iy * kVqGrid + ix, the ascending indices of the only
// codewords that can be nearest to a point of the cell (the last repeated),
// or 0xFF in byte 0 when more than four can be.
constexpr int kVqGridLog = 6;
constexpr int kVqGrid = 1 << kVqGridLog;
constexpr int kVqGridMaxN = 64;

}  // namespace tq

struct tq_codebook {
    tq_spec spec;
    bool dense;
    int K;
    int device;
    std::vector<float> levels, thresholds, rotation, sketch;  // host mirrors
    std::vector<float> mu;  // sign correction: per KV head (or one shared), else empty
    void* block = nullptr;                                    // one device allocation
    tq::DeviceTables dev;
    // levels in 24-bit fixed point, t_k ~= T_k * 2^-lvl_shift, as three balanced
    // base-256 int8 digits (digit 0 most significant); word 2b holds digit b
    // of codes 0..3, word 2b+1 of codes 4..7 (byte tables for v_perm)
    uint32_t lvl_digits[16] = {};
    int lvl_shift = 0;
    // vector codebooks (block 2, N <= 64): the encoder's candidate grid
    std::vector<uint32_t> vq_grid;
    float vq_inv_cell = 0.0f;
};

namespace tq {

inline bool sign_corr(const tq_codebook* cb) { return cb->spec.correction == TQ_CORR_SIGN; }
inline bool no_rotation(const tq_codebook* cb) { return cb->spec.rotation == TQ_ROT_NONE; }
// scale of the correction term: sqrt(pi/2)/m for the QJL sketch, 1 for the
// sign correction (whose mu is applied per KV head)
inline double corr_scale(const tq_codebook* cb) {
    if (sign_corr(cb)) return 1.0;
    return cb->spec.m ? 1.2533141373155003 / (double)cb->spec.m : 0.0;
}
// planes a record of this codebook carries
inline bool has_rnorm(const tq_codebook* cb) { return cb->spec.m > 0 && !sign_corr(cb); }
// mu of KV head kh on the device (sign correction), else nullptr; the
// stride is 0 for one shared value
struct MuRef {
    const float* ptr = nullptr;
    int stride = 0;
};
inline MuRef mu_ref(const tq_codebook* cb) {
    MuRef r;
    if (sign_corr(cb)) {
        r.ptr = cb->dev.mu;
        r.stride = cb->mu.size() > 1 ? 1 : 0;
    }
    return r;
}

// ---- error reporting (thread-local message, see tq_last_error) ----
tq_status fail(tq_status code, const std::string& msg);
tq_status hip_fail(hipError_t e, const char* what);

// ---- host math (tq_host.cpp) ----
tq_status check_spec(const tq_spec& s, bool* dense);
void lloyd_max_table(int d, int bits, std::vector<double>* levels, std::vector<double>* thr);
double beta_mean_abs_error(int d, const std::vector<float>& levels, const std::vector<float>& thr);
void fibquant_codebook(int d, int k, int N, std::vector<double>* code);  // [N][k] row-major
void splitmix_gaussians(uint64_t seed, int purpose, size_t n, double* out);
void splitmix_signs(uint64_t seed, size_t n, int8_t* out);
void haar_from_gaussians(int d, const double* g, std::vector<double>* q);  // row-major
void level_digits(const std::vector<float>& levels, uint32_t words[16], int* shift);
uint16_t f32_to_f16(float f);
float f16_to_f32(uint16_t h);

// ---- kernel launchers (tq_encode.hip, tq_attn.hip, tq_gemm.hip) ----
// paged records: table [B][max_pages] of physical pages of `size` slots
// (table == nullptr: contiguous records of L_cap slots per (sequence, head))
struct PageRef {
    const int32_t* table = nullptr;
    int32_t size = 0, max_pages = 0;
    int64_t n_pages = 0;
};
struct EncodeArgs {
    const void* x;
    int64_t s_seq, s_tok, s_head;
    int32_t n_seq, n_tok, h_kv, tok_offset, L_cap;
    int32_t bf16;
    const float* rope_cos;  // nullptr: no RoPE
    const float* rope_sin;
    tq_packed out;
    void* ws;  // dense form only
    size_t ws_bytes;
    int32_t append = 0;           // one token per (sequence, head) at slot pos[sequence]
    const int32_t* pos = nullptr;
    int32_t rope_npos = 0;
    PageRef pages;
};
hipError_t launch_encode(const tq_codebook* cb, const EncodeArgs& a, hipStream_t stream);
size_t encode_workspace_bytes(const tq_codebook* cb, int64_t n_vectors);

struct AttnArgs {
    const void* q;
    int32_t bf16;
    int32_t B, Hq, h_kv, L_cap;
    const int32_t* seq_len;
    const int32_t* q_pos;  // RoPE position of each sequence's query (nullptr: seq_len)
    const float* rope_cos;
    const float* rope_sin;
    float scale;
    int32_t top_k;
    float* out;
    int32_t* topk_idx;
    void* ws;
    size_t ws_bytes;
    PageRef pages;
};
hipError_t launch_logits(const tq_codebook* ck, const tq_packed& k, const AttnArgs& a,
                         hipStream_t stream);
hipError_t launch_decode(const tq_codebook* ck, const tq_codebook* cv, const tq_packed& k,
                         const tq_packed& v, const AttnArgs& a, hipStream_t stream);
size_t logits_workspace_bytes(const tq_codebook* ck, int64_t B, int Hq, int h_kv, int L_cap,
                              int top_k);
size_t decode_workspace_bytes(const tq_codebook* ck, const tq_codebook* cv, int64_t B, int Hq,
                              int h_kv, int L_cap);

// Fixed-point digit form of prepared queries (tq_qprep.hip).
struct QDigits {
    float* qp;      // [rows][d]   q' = Pi RoPE(q)
    float* s;       // [rows][m]   s = S q'
    int8_t* qd;     // [rows*4][d] balanced base-128 digits of q' (most significant first)
    int8_t* sd;     // [rows*4][sdw] digits of s in MFMA slot order
    float* scale;   // [rows][3]   shift(q'), shift(s) (x ~= X * 2^-shift), fixed-point sum of s
    int sdw, ncs;
};
bool logits_mfma_supported(const tq_codebook* ck);
size_t qdigits_workspace_bytes(const tq_codebook* ck, int64_t rows);
QDigits carve_qdigits(const tq_codebook* ck, void* ws, int64_t rows);
hipError_t launch_qdigits(const tq_codebook* ck, const AttnArgs& a, const QDigits& q, hipStream_t stream);
// the integer-MFMA logit scan (tq_scan.hip): query rows in tiles of four;
// where scan_prepares_queries (q == nullptr) each workgroup prepares its own
// queries, elsewhere it reads those launch_qdigits prepared
bool scan_supported(const tq_codebook* ck);
int scan_row_tiles(int G);
bool scan_prepares_queries(const tq_codebook* ck, int G);  // the scan prepares the queries itself (no query workspace)
hipError_t launch_scan(const tq_codebook* ck, const tq_packed& k, const AttnArgs& a, const QDigits* q, int k0,
                       int klen, float* out, int64_t ld, int col0, hipStream_t stream);
// Fused decode on the integer matrix cores (tq_decode.hip): partials of
// [B*Hq][nsplit][2 + d + m] floats (max, sum, A_y, A_z) for the merge kernel.
bool decode_mfma_supported(const tq_codebook* ck, const tq_codebook* cv);
void decode_mfma_plan(int64_t B, int Hq, int h_kv, int L_cap, int* nsplit, int* split_len);
hipError_t launch_decode_mfma(const tq_codebook* ck, const tq_codebook* cv, const tq_packed& k, const tq_packed& v,
                              const AttnArgs& a, const QDigits& q, float* part, int nsplit, int split_len,
                              hipStream_t stream);

// FibQuant vector codebooks (tq_vq.hip): block 2, Hadamard rotation, d = 64, 128
bool vq_supported(const tq_codebook* cb);
hipError_t launch_vq_logits(const tq_codebook* ck, const tq_packed& k, const AttnArgs& a, const float* qp, int k0,
                            int klen, float* out, int64_t ld, int col0, hipStream_t stream);
// fused decode with vector-coded keys and values (Hadamard, d = 64 or 128):
// the split kernel writes (M, l, A_y) partials for the split merge
bool vq_attn_supported(const tq_codebook* ck, const tq_codebook* cv);
void vq_attn_plan(int L_cap, int* nsplit, int* split_len);
hipError_t launch_vq_attn_split(const tq_codebook* ck, const tq_codebook* cv, const tq_packed& k, const tq_packed& v,
                                const AttnArgs& a, const float* qp, float* part, int nsplit, int split_len,
                                hipStream_t stream);
hipError_t launch_vq_decode(const tq_codebook* cb, const tq_packed& k, int64_t first, int64_t count, float* out,
                            hipStream_t stream);
hipError_t launch_qprep_rht(const tq_codebook* ck, const AttnArgs& a, float* qp, float* s, hipStream_t stream);
hipError_t launch_topk(const AttnArgs& a, const float* scores, int64_t ld, int64_t row0, int col0, int cnt,
                       bool first, hipStream_t stream);

// C[M][N] = A[M][K] * B[N][K]^T, fp32, row-major with leading dimensions
// lda/ldb/ldc (elements).
hipError_t launch_gemm_nt(const float* A, int64_t lda, const float* B, int64_t ldb, float* C,
                          int64_t ldc, int M, int N, int K, hipStream_t stream);
// Index-scan scores against packed scalar records: row n of B is key
// rec0 + n's rotated-domain estimate [t[c_0..c_{d-1}], sqrt(pi/2)/m gamma
// (+-1)_0..m-1] (d and m multiples of 32, 1, 2 or 4 bits), A = [q' | s] split
// beforehand by launch_split_rows into three bf16 piece planes [3][rows][d + m].
struct RecB {
    const uint32_t* codes;
    const uint32_t* signs;
    const float* rnorm;
    const float* levels;
    int64_t rec0;
    int32_t d, m, bits;
};
bool gemm_records_supported(int d, int m, int bits);
size_t gemm_records_split_bytes(int64_t M, int d, int m);
hipError_t launch_split_rows(const float* A, int64_t lda, int M, int K, void* planes, hipStream_t stream);
// planes: the M rows' first piece (`plane` elements between pieces)
hipError_t launch_gemm_records(const void* planes, int64_t plane, int M, const RecB& rec, float* C, int64_t ldc,
                               int N, hipStream_t stream);

}  // namespace tq
