/*
 * tq.h - C ABI of libtq, an MI355X (gfx950) implementation of the hot path
 * of a TurboQuant-style KV-cache codec: normalise-rotate-quantise encoding
 * with a one-bit QJL sketch of the residual, and decode-time attention
 * computed straight from the packed records.
 *
 * Sources (by page title and section):
 *   FibQuant summary ("FibQuant: Quantizacao Vetorial Universal para
 *     Compressao de KV-Cache de Acesso Aleatorio"), section 1: a deployable
 *     cache codec stores fixed-rate records at fixed addresses so any token
 *     decodes on its own; the interface stores the norm, applies one shared
 *     random rotation and quantises each rotated coordinate with a scalar
 *     Lloyd-Max table.  Section 2.1: one offline table serves every layer,
 *     head and input.  Section 2.3: decoding looks up codes, applies the
 *     inverse rotation and scales by the norm.
 *   iaemfoco post ("TurboQuant: Compressao Avancada da Google para Cache KV
 *     ..."), section "TurboQuant: Uma Nova Abordagem": a randomized Hadamard
 *     rotation, then a quantized Johnson-Lindenstrauss step that makes inner
 *     products unbiased.
 *   itstec post ("Compressao KV eficaz com TurboQuant"), section "Por dentro
 *     do processo de compressao KV": the residual's JL projection is kept as
 *     sign bits only.
 *   TurboESM summary, technical section 2: RoPE before the rotation; a fused
 *     decode kernel (dequantisation, residual correction, online softmax)
 *     with no intermediate dequantised copy.
 *   tambur post ("Google acelera LLMs em 8 vezes"): attention logits
 *     computed from quantised keys.
 *   TurboESM summary, technical section 2, also: separate 8-entry tables
 *     for keys (rotated) and values (original coordinates), and a one-bit
 *     sign per residual coordinate corrected by a calibrated mean residual
 *     magnitude (the TQ_CORR_SIGN codebooks below).
 *
 * Conventions for every entry point
 *   - Device pointers are HIP device memory owned by the caller; host
 *     pointers are ordinary host memory owned by the caller.  The library
 *     owns only a codebook's tables (tq_codebook_init / tq_codebook_destroy)
 *     and never allocates in encode, logits or decode calls: scratch space is
 *     the caller's workspace, sized by tq_workspace_bytes().
 *   - Arguments are validated on the host before anything is launched; an
 *     invalid call returns an error code and launches nothing.  Work is
 *     enqueued on `stream` (a hipStream_t; NULL = the default stream) and
 *     the call returns without synchronising.  A failed launch returns
 *     TQ_EHIP.  tq_last_error() gives a message for the calling thread's
 *     last failure.
 *   - Outputs must not alias inputs.  Calls that write the same buffers
 *     must be ordered by the caller (same stream or events).
 *   - Non-finite inputs give unspecified (but bounded, non-faulting) output.
 *
 * Packed record (one set of planes per tensor; vector index
 * n = (seq * h_kv + head) * L_cap + token):
 *   norm [n]          float    nu = ||x||_2 (after RoPE for keys)
 *   rnorm[n]          float    gamma = ||y - t[c]||_2 (absent when m == 0
 *                              and for TQ_CORR_SIGN codebooks)
 *   (vector codebooks: codes[n][ceil(bits * d / block / 32)], the index of
 *   block j at bits [j*bits, (j+1)*bits) LSB first; no rnorm or signs)
 *   codes[n][b*d/32]  uint32   code 0 is the most negative level; bit k of
 *                              the words' bit string is bit k%32 of word k/32.
 *                              b = 1, 2, 4: coordinate i's code is bits
 *                              [b*i, b*i+b).  b = 3: coordinates in groups of
 *                              32 take words 3g..3g+2 (W0..W2); coordinate
 *                              j < 24 of a group is bits 8(j%4) + 3((j%8)/4)
 *                              .. +2 of W_{j/8}; for j = 24 + r the low two
 *                              bits are bits 8(r%4)+6, +7 of W_{r/4} and the
 *                              high bit is bit 8(r%4) + 6 + r/4 of W2
 *   signs[n][m/32]    uint32   bit l (bit l%32 of word l/32) is 1 iff
 *                              (S e)_l >= 0; for TQ_CORR_SIGN (S = I,
 *                              m = d) iff e_l >= 0
 * A TQ_CORR_SIGN record at d = 64, b = 3 is 4 + 24 + 8 = 36 bytes.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t tq_status;
enum {
    TQ_OK = 0,
    TQ_EINVAL = -1,        /* bad argument (null pointer, size, stride, alignment) */
    TQ_EUNSUPPORTED = -2,  /* valid spec the library has no kernel for */
    TQ_ENOMEM = -3,        /* device allocation failed (codebook init only) */
    TQ_EHIP = -4           /* a HIP runtime call or kernel launch failed */
};

enum { TQ_F32 = 0, TQ_BF16 = 1 };                                  /* element types */
enum { TQ_ROT_AUTO = 0, TQ_ROT_HADAMARD = 1, TQ_ROT_DENSE = 2, TQ_ROT_NONE = 3 };  /* rotation forms */
enum { TQ_CORR_QJL = 0, TQ_CORR_SIGN = 1 };                        /* residual corrections */
enum { TQ_OP_ENCODE = 0, TQ_OP_LOGITS = 1, TQ_OP_DECODE = 2 };     /* workspace queries */

/*
 * Codebook specification.
 *   d        vector dimension.  Hadamard form: 64 or 128.  Dense form: a
 *            multiple of 64 up to 4096.
 *   bits     Lloyd-Max bits per coordinate, 1..4 (K = 2^bits levels);
 *            bits*d must be a multiple of 32.
 *   m        QJL sketch rows: 0 (no sketch, no rnorm plane) or a multiple of
 *            32 up to 4096; the Hadamard form has kernels for m = 0, d/2, d.
 *   rotation TQ_ROT_AUTO (Hadamard iff d is a power of two), _HADAMARD,
 *            _DENSE, or _NONE (Pi = I: vectors quantised in their original
 *            coordinates; TQ_CORR_SIGN codebooks only).
 *   seed     draws sigma, the rotation Gaussians and S when no tq_draws are
 *            given (SplitMix64 streams, Box-Muller Gaussians).
 *   correction
 *            TQ_CORR_QJL (0): S is an m x d Gaussian sketch, gamma is stored
 *            and the correction is sqrt(pi/2)/m gamma S^T z.
 *            TQ_CORR_SIGN (TurboESM summary, technical section 2): one sign
 *            per residual coordinate (S = I, so m must equal d), no gamma
 *            plane, and the correction is mu z with mu the codebook's mean
 *            residual magnitude of the record's KV head.  Needs d = 64 or
 *            128, bits 1..3, rotation Hadamard or none.
 *   block    0 or 1: a scalar Lloyd-Max table per coordinate (the above).
 *            2 or 3: a FibQuant vector codebook (FibQuant summary, section
 *            2): N = 2^bits codewords (bits 1..8) for blocks of `block`
 *            consecutive rotated coordinates, built offline for the
 *            spherical-Beta law of such a block (Bennett-Gersho radii,
 *            golden-spiral / Fibonacci-sphere directions, Lloyd-Max with
 *            restarts); rate bits / block per coordinate.  m must be 0,
 *            correction TQ_CORR_QJL (no residual correction) and d a multiple
 *            of block.  Kernels exist for block 2 with the Hadamard rotation
 *            (d = 64, 128), and for block 2 or 3 with a dense rotation (d a
 *            multiple of 64: bulk encodes and contiguous scans; appends and
 *            pages return TQ_EUNSUPPORTED); other vector codebooks build
 *            tables only.
 */
typedef struct {
    int32_t d, bits, m, rotation;
    uint64_t seed;
    int32_t correction, block;
} tq_spec;

/*
 * Explicit random draws (host memory, read during the call only).  Any
 * field may be NULL; NULL fields are derived from spec->seed.
 *   sigma     [d] int8 +1/-1   Hadamard form: Pi = H diag(sigma) / sqrt(d)
 *   rot_gauss [d*d] double     dense form: Pi = Q of rot_gauss = Q R with
 *                              diag(R) > 0, stored as float32 (row-major,
 *                              y = Pi u)
 *   sketch    [m*d] float      S, row-major (must be NULL for
 *                              TQ_CORR_SIGN, whose S is the identity)
 * TQ_ROT_NONE codebooks read no sigma.
 */
typedef struct {
    const int8_t* sigma;
    const double* rot_gauss;
    const float* sketch;
} tq_draws;

typedef struct tq_codebook tq_codebook;  /* opaque; immutable after init */

/* Caller-owned planes of one packed tensor (device memory); n = capacity in
 * records.  rnorm and signs may be NULL when the codebook has m == 0; rnorm
 * may be NULL for TQ_CORR_SIGN codebooks (it is neither read nor written). */
typedef struct {
    float* norm;
    float* rnorm;
    uint32_t* codes;
    uint32_t* signs;
    int64_t n;
} tq_packed;

/*
 * Paged records (FibQuant summary, section 1: fixed addresses, any token
 * decodable by address arithmetic; TurboESM summary, technical section 5:
 * autoregressive generation).  A sequence's cache slots are cut into pages
 * of page_size slots; pages[b * max_pages + j] is the physical page that
 * holds logical page j of sequence b, and physical page p holds every KV
 * head's slots: the record of (b, head, slot t) is
 *     n = (pages[b][t / page_size] * h_kv + head) * page_size + t % page_size.
 *   pages      device int32 [B][max_pages], owned by the caller
 *   page_size  a positive multiple of 64
 *   max_pages  row length; max_pages * page_size < 2^31 (the logical capacity)
 *   n_pages    physical pages; record planes hold n_pages * h_kv * page_size
 *              records.  Entries outside [0, n_pages) are never dereferenced:
 *              encodes skip such slots, scans read page 0 or n_pages - 1
 *              instead (the caller keeps every entry below seq_len valid).
 */
typedef struct {
    const int32_t* pages;
    int32_t page_size, max_pages;
    int64_t n_pages;
} tq_pages;

/*
 * tq_codebook_tables (host only, no GPU): computes the tables a codebook
 * holds, into caller host buffers (any may be NULL to skip):
 *   (vector codebooks: levels receives the N x block codewords row-major,
 *   thresholds nothing)
 *   levels [K], thresholds [K-1]    float32 Lloyd-Max table for the density
 *       of one coordinate of a uniform point on S^{d-1} (FibQuant summary,
 *       section 2.1; itstec post, "Por dentro do processo": a Beta law),
 *       levels at the conditional means, thresholds at the midpoints
 *   rotation  Hadamard: [d] sigma as +-1.0f; dense: [d*d] Pi row-major; none: not written
 *   sketch    [m*d] S row-major (the identity for TQ_CORR_SIGN)
 * Returns TQ_EINVAL / TQ_EUNSUPPORTED for a bad spec.
 */
tq_status tq_codebook_tables(const tq_spec* spec, const tq_draws* draws, float* levels,
                             float* thresholds, float* rotation, float* sketch);

/*
 * tq_codebook_init: builds the tables (as tq_codebook_tables) and uploads
 * them to the current HIP device on `stream` (the only host-to-device copy
 * the library makes).  *out receives a handle owned by the library.
 * Errors: TQ_EINVAL (null out/spec, bad spec), TQ_EUNSUPPORTED,
 * TQ_ENOMEM, TQ_EHIP.  On error *out is set to NULL.
 */
tq_status tq_codebook_init(const tq_spec* spec, const tq_draws* draws, void* stream,
                           tq_codebook** out);

/*
 * tq_codebook_init_calibrated: as tq_codebook_init, with the table and (for
 * TQ_CORR_SIGN) the mean residual magnitudes given instead of derived
 * (TurboESM summary, technical section 2: per-tensor tables and a
 * calibrated residual magnitude; see tq_calibrate).
 *   levels   host float [2^bits], strictly increasing and symmetric
 *            (levels[K-1-j] == -levels[j] exactly), or NULL for the
 *            spherical-Beta Lloyd-Max table.  Thresholds are the midpoints
 *            of neighbouring levels, formed in double and rounded to float.
 *   mu, n_mu host float [n_mu], finite and >= 0: mu of KV head h is
 *            mu[n_mu == 1 ? 0 : h]; calls on the codebook then need
 *            h_kv == n_mu unless n_mu == 1.  NULL (n_mu 0) gives one shared
 *            mu = E|Y - t[c(Y)]| under the spherical-Beta law of the table.
 *            Must be NULL / 0 for TQ_CORR_QJL codebooks.
 * Errors as tq_codebook_init, and TQ_EINVAL for a bad table or mu.
 */
tq_status tq_codebook_init_calibrated(const tq_spec* spec, const tq_draws* draws, const float* levels,
                                      const float* mu, int32_t n_mu, void* stream, tq_codebook** out);

/*
 * tq_calibrate (host only, no GPU): fits a TQ_CORR_SIGN codebook's table
 * and per-head mean residual magnitudes to a calibration batch (TurboESM
 * summary, technical section 2).
 *   x          host float [n_tok][h][d] (contiguous): vectors as the encoder
 *              would receive them; token t sits at position tok_offset + t
 *   rope_cos, rope_sin, rope_npos   host tables as tq_rope_table writes
 *              them ([rope_npos][d/2]), or NULL for no RoPE; they must
 *              cover position tok_offset + n_tok - 1
 *   levels     out: host float [2^bits], the symmetric table: its upper
 *              half is Lloyd's fixed point for |y| over every head's rotated
 *              unit vectors (y = Pi RoPE(x) / nu, vectors with nu = 0 left
 *              out), started from the order statistics
 *              |y|_(floor((j + 1/2) N / (K/2))) of the N sorted values and
 *              iterated until no value changes cell (a value on a boundary
 *              goes to the upper cell; an empty cell keeps its level)
 *   mu         out: host float [h], mean |y_i - t[c_i]| over head h's
 *              vectors and coordinates, codes decided in float against the
 *              float table (0 for a head with no non-zero vector)
 * The rotation is the one spec/draws give (sigma for Hadamard, identity for
 * TQ_ROT_NONE).  Errors: TQ_EINVAL (bad spec or sizes, no non-zero vector),
 * TQ_EUNSUPPORTED.
 */
tq_status tq_calibrate(const tq_spec* spec, const tq_draws* draws, const float* x, int64_t n_tok,
                       int32_t h, int32_t tok_offset, const float* rope_cos, const float* rope_sin,
                       int32_t rope_npos, float* levels, float* mu);

/* The codebook's mean residual magnitudes: *n_mu receives their count (0 for
 * TQ_CORR_QJL), mu (host float [*n_mu], may be NULL) the values. */
tq_status tq_codebook_get_mu(const tq_codebook* cb, float* mu, int32_t* n_mu);

/* Frees a codebook's device tables.  The caller guarantees no enqueued
 * work still uses it (synchronise first).  NULL is accepted. */
tq_status tq_codebook_destroy(tq_codebook* cb);

/* Copies the spec the codebook was built with. */
tq_status tq_codebook_get_spec(const tq_codebook* cb, tq_spec* out);

/* Host copies of the codebook's tables (same layout as tq_codebook_tables). */
tq_status tq_codebook_export(const tq_codebook* cb, float* levels, float* thresholds,
                             float* rotation, float* sketch);

/*
 * tq_encode_kv: encodes keys and/or values into packed records (FibQuant
 * summary, sections 1 and 2.3; iaemfoco post, "Uma Nova Abordagem"; itstec
 * post, "Por dentro do processo"; TurboESM summary, technical section 2 for
 * RoPE first).  Per vector: RoPE (keys only, if tables are given) -> nu ->
 * y = Pi (x / nu) -> codes -> residual e = y - t[c], gamma = ||e|| ->
 * sign bits of S e.
 *   ck, k, kout   key codebook, input and planes (k may be NULL: no keys)
 *   cv, v, vout   value codebook, input and planes (v may be NULL)
 *   dtype         TQ_F32 or TQ_BF16 for both inputs
 *   n_seq, n_tok, h_kv   input shape [n_seq][n_tok][h_kv][d]; d contiguous
 *   k_stride, v_stride   host int64[3]: element strides of seq, tok, head;
 *                 each a multiple of 4 (f32) or 8 (bf16), base pointers
 *                 16-byte aligned
 *   tok_offset    cache slot (and RoPE position) of token 0
 *   L_cap         cache capacity per (seq, head); tok_offset + n_tok <= L_cap
 *   rope_cos, rope_sin   device float [rope_npos][d/2] (see tq_rope_table)
 *                 or both NULL for no RoPE; tok_offset + n_tok <= rope_npos
 *   ws, ws_bytes  device workspace, at least tq_workspace_bytes(ck, cv,
 *                 TQ_OP_ENCODE, n_seq*n_tok*h_kv, ...) (0 for Hadamard codebooks)
 * n_seq*n_tok*h_kv == 0 is a no-op returning TQ_OK.  Hadamard codebooks
 * take at most 2^31 - 1 tiles of 32 tokens x 1 head per call
 * (TQ_EUNSUPPORTED beyond).
 */
tq_status tq_encode_kv(const tq_codebook* ck, const tq_codebook* cv, const void* k, const void* v,
                       int32_t dtype, int32_t n_seq, int32_t n_tok, int32_t h_kv,
                       const int64_t* k_stride, const int64_t* v_stride, int32_t tok_offset,
                       int32_t L_cap, const float* rope_cos, const float* rope_sin,
                       int32_t rope_npos, const tq_packed* kout, const tq_packed* vout, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * tq_encode_kv_paged: as tq_encode_kv, into paged records: slot
 * tok_offset + t of sequence s goes through the page table (tok_offset +
 * n_tok <= max_pages * page_size).  Hadamard and unrotated codebooks only
 * (TQ_EUNSUPPORTED for dense ones); no workspace.
 */
tq_status tq_encode_kv_paged(const tq_codebook* ck, const tq_codebook* cv, const void* k, const void* v,
                             int32_t dtype, int32_t n_seq, int32_t n_tok, int32_t h_kv, const int64_t* k_stride,
                             const int64_t* v_stride, int32_t tok_offset, const tq_pages* pages,
                             const float* rope_cos, const float* rope_sin, int32_t rope_npos,
                             const tq_packed* kout, const tq_packed* vout, void* stream);

/*
 * tq_append_kv: one autoregressive step's keys and/or values, one token per
 * (sequence, KV head), each sequence at its own slot (FibQuant summary,
 * section 1: a record at a fixed address; TurboESM summary, technical
 * section 5: autoregressive generation).  The token of sequence b goes to
 * slot pos[b], which is also its RoPE position.
 *   k, v          device [B][h_kv][d] (dtype as tq_encode_kv), strides
 *                 host int64[2] (sequence, head) in elements, multiples of
 *                 16 bytes
 *   pos           device int32 [B]; a slot outside the cache (or behind a
 *                 page entry outside the pool) is encoded but not stored
 *   pages         paged records, or NULL for contiguous records of L_cap
 *                 slots per (sequence, head)
 *   rope_*        as tq_encode_kv; every pos[b] must be below rope_npos
 *                 (a position beyond the table reads its last row)
 * Hadamard and unrotated codebooks only.  Writes nothing but the records of
 * the B * h_kv appended tokens.
 */
tq_status tq_append_kv(const tq_codebook* ck, const tq_codebook* cv, const void* k, const void* v, int32_t dtype,
                       int32_t B, int32_t h_kv, const int64_t* k_stride, const int64_t* v_stride,
                       const int32_t* pos, const tq_pages* pages, int32_t L_cap, const float* rope_cos,
                       const float* rope_sin, int32_t rope_npos, const tq_packed* kout, const tq_packed* vout,
                       void* stream);

/*
 * tq_attn_logits: attention logits from packed keys (tambur post; iaemfoco
 * post, "Uma Nova Abordagem" for the unbiased QJL correction):
 *   logit[b][h][t] = nu_t ( <q'_h, t[c_t]> + sqrt(pi/2)/m gamma_t <s_h, z_t> )
 * with q'_h = Pi RoPE(q_h, seq_len[b]), s_h = S q'_h, z in {-1,+1}; for a
 * TQ_CORR_SIGN codebook the second term is mu_kv <q'_h, z_t> (TurboESM
 * summary, technical section 2), kv = h / (Hq / h_kv).
 *   q             device [B][Hq][d], dtype TQ_F32 or TQ_BF16
 *   k             packed keys, capacity >= B*h_kv*L_cap
 *   B, Hq, h_kv   Hq a multiple of h_kv; query head h reads KV head h/(Hq/h_kv)
 *   seq_len       device int32 [B]; keys t < seq_len[b] are scored (values
 *                 above L_cap are clamped to L_cap)
 *   q_pos         device int32 [B]: the RoPE position of sequence b's query,
 *                 or NULL for seq_len[b] (a query whose own key is not yet in
 *                 the cache).  A decode step that appended its token's key at
 *                 slot p before scoring passes q_pos = p with seq_len = p + 1,
 *                 so that the query and its own key share a position.
 *                 Clamped to [0, L_cap] like seq_len.
 *   rope_*        as tq_encode_kv (rope_npos > L_cap) or NULL
 *   top_k = 0     out = device float [B][Hq][L_cap]; entries t >= seq_len[b]
 *                 are left untouched
 *   top_k = 1..16 out = device float [B][Hq][top_k] best logits in
 *                 descending order (ties to the smaller index), topk_idx =
 *                 device int32 [B][Hq][top_k] (-1 / -inf when fewer keys)
 *   ws, ws_bytes  device workspace >= tq_workspace_bytes(ck, NULL,
 *                 TQ_OP_LOGITS, B, Hq, h_kv, L_cap, top_k)
 */
tq_status tq_attn_logits(const tq_codebook* ck, const void* q, int32_t q_dtype, const tq_packed* k,
                         int32_t B, int32_t Hq, int32_t h_kv, int32_t L_cap, const int32_t* seq_len,
                         const int32_t* q_pos, const float* rope_cos, const float* rope_sin, int32_t rope_npos,
                         int32_t top_k, float* out, int32_t* topk_idx, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * tq_attn_decode: fused decode attention over packed K and V (TurboESM
 * summary, technical section 2, fused kernel; FibQuant summary, section 2.3
 * for value reconstruction):
 *   out[b][h] = sum_t p_t nu^v_t Pi_v^T (t_v[c^v_t] + sqrt(pi/2)/m_v gamma^v_t S_v^T z^v_t),
 *   p = softmax over t < seq_len[b] of scale * logit[b][h][t];
 * a TQ_CORR_SIGN value codebook takes mu_kv z^v_t as the correction term
 * (and Pi_v = I for TQ_ROT_NONE).  Scalar key and value codebooks need the
 * same d, bits and m and a Hadamard or no rotation (TQ_EUNSUPPORTED before
 * any launch otherwise); TQ_CORR_SIGN codebooks are served for bits <= 3 only.
 * Vector codebooks (FibQuant summary, sections 2.3 and 5) are served for
 * keys and values together - block 2, Hadamard, d = 64 or 128, at most 5
 * key index bits at d = 128 (6 at d = 64), values of any size - with
 * out = sum_t p_t nu^v_t Pi_v^T (c_v[idx^v_t(0)], c_v[idx^v_t(1)], ...) and the
 * logit nu^k_t <q', concatenated key codewords>; mixing scalar and vector
 * codebooks, or more than 65535 splits of 256 keys, is TQ_EUNSUPPORTED.
 * Split over the key axis with an online softmax and a log-sum-exp merge.
 *   scale         0 means 1/sqrt(d)
 *   out           device float [B][Hq][d]; zeros where seq_len[b] == 0
 *   other arguments as tq_attn_logits; ws >= tq_workspace_bytes(ck, cv,
 *   TQ_OP_DECODE, B, Hq, h_kv, L_cap, 0)
 */
tq_status tq_attn_decode(const tq_codebook* ck, const tq_codebook* cv, const void* q, int32_t q_dtype,
                         const tq_packed* k, const tq_packed* v, int32_t B, int32_t Hq, int32_t h_kv,
                         int32_t L_cap, const int32_t* seq_len, const int32_t* q_pos, const float* rope_cos,
                         const float* rope_sin, int32_t rope_npos, float scale, float* out,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * tq_attn_decode_noalloc: tq_attn_decode for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and result as tq_attn_decode without ws and
 * ws_bytes: the workspace is a static device array of the library, 32 MiB
 * on every GPU the library runs on, held until the process ends.  The call
 * allocates nothing.  A decode whose tq_workspace_bytes(ck, cv,
 * TQ_OP_DECODE, ...) exceeds the array is refused with TQ_EINVAL before any
 * launch.  Every call on one GPU shares that GPU's array (it keeps the last
 * call's contents; the decode writes every scratch byte it reads), so calls
 * that overlap on one GPU - on two streams at once - race.
 */
tq_status tq_attn_decode_noalloc(const tq_codebook* ck, const tq_codebook* cv, const void* q, int32_t q_dtype,
                                 const tq_packed* k, const tq_packed* v, int32_t B, int32_t Hq, int32_t h_kv,
                                 int32_t L_cap, const int32_t* seq_len, const int32_t* q_pos,
                                 const float* rope_cos, const float* rope_sin, int32_t rope_npos, float scale,
                                 float* out, void* stream);

/*
 * Paged forms of tq_attn_logits and tq_attn_decode: keys (and values) are
 * read through the page table; the logical capacity max_pages * page_size
 * takes the place of L_cap (logit rows are [max_pages * page_size] wide,
 * workspaces are sized with it).  Bits <= 4 Hadamard or unrotated scalar
 * codebooks, or Hadamard vector codebooks (TQ_EUNSUPPORTED otherwise).
 */
tq_status tq_attn_logits_paged(const tq_codebook* ck, const void* q, int32_t q_dtype, const tq_packed* k, int32_t B,
                               int32_t Hq, int32_t h_kv, const int32_t* seq_len, const int32_t* q_pos,
                               const tq_pages* pages, const float* rope_cos, const float* rope_sin, int32_t rope_npos,
                               int32_t top_k, float* out, int32_t* topk_idx, void* ws, size_t ws_bytes, void* stream);
tq_status tq_attn_decode_paged(const tq_codebook* ck, const tq_codebook* cv, const void* q, int32_t q_dtype,
                               const tq_packed* k, const tq_packed* v, int32_t B, int32_t Hq, int32_t h_kv,
                               const int32_t* seq_len, const int32_t* q_pos, const tq_pages* pages,
                               const float* rope_cos, const float* rope_sin, int32_t rope_npos, float scale,
                               float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * tq_decode_vectors: the FibQuant decoder (FibQuant summary, section 2.3):
 * records [first, first + count) of a vector-coded tensor rebuilt as
 * out[i] = nu Pi^T (c[idx_0], c[idx_1], ...) (device float [count][d]).
 * Vector codebooks with kernels only (TQ_EUNSUPPORTED otherwise).  Values
 * the fused decode (tq_attn_decode) does not serve - a dense rotation, or
 * scalar keys with vector-coded values - are rebuilt here.
 */
tq_status tq_decode_vectors(const tq_codebook* cb, const tq_packed* packed, int64_t first, int64_t count, float* out,
                            void* stream);

/* Workspace bytes for an op.  For TQ_OP_ENCODE pass the vector count in B
 * (other sizes ignored).  Returns 0 on a bad argument. */
size_t tq_workspace_bytes(const tq_codebook* ck, const tq_codebook* cv, int32_t op, int64_t B,
                          int32_t Hq, int32_t h_kv, int32_t L_cap, int32_t top_k);

/* uint32 words per record of a plane: plane 0 = codes (bits*d/32),
 * plane 1 = signs (m/32).  -1 on a bad spec. */
int64_t tq_plane_words(const tq_spec* spec, int32_t plane);

/* Host RoPE table: cos/sin[pos][i] = cos/sin(pos * base^(-2i/d)), angles in
 * double, stored as float (i < d/2, pos < n_pos).  Half-split pairing: RoPE
 * rotates (x_i, x_{i+d/2}).  cos_out and sin_out are host float[n_pos*d/2]. */
tq_status tq_rope_table(double base, int32_t d, int32_t n_pos, float* cos_out, float* sin_out);

/* Message for the calling thread's last failed call ("" if none). */
const char* tq_last_error(void);

/* Library version string. */
const char* tq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H */
