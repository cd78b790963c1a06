/*
 * ispa.h - C ABI of the ISPA hot path on AMD Instinct MI355X (gfx950).
 *
 * ISPA = Instance-Specific Parametric Absorption, from the paper "Towards
 * Memory-Efficient Autoregressive Video Generation via Instance-Specific
 * Parametric Absorption". During a short warmup every attention layer runs
 * as a full-history layer while the local-only output (sink frame + current
 * frames) is collected beside it (§3.1 item 1, §3.4). At the end of warmup a
 * closed-form least-squares update dW of each layer's output projection is
 * fitted so that the local output through W + dW reproduces the full output
 * through W (§3.1 item 2, §3.2, ridge parameter of §4.1); layers are ranked
 * by their reconstruction error and the K best take the update in place and
 * drop their history KV (§3.3). L-layers then run local attention only with
 * W + dW (§3.1 item 3).
 *
 * Conventions for every entry point:
 *  - Pointers are device pointers unless stated otherwise; the caller owns
 *    every buffer. The library never allocates, frees or synchronises, with
 *    the one exception of the streaming KV cache (ispa_kv_*), which owns the
 *    KV memory it manages.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and the call returns immediately. Argument checks are synchronous: on
 *    any error status nothing has been enqueued.
 *  - bf16 tensors are passed as raw 16-bit storage (void*).
 *  - Row-major, contiguous. Weight-shaped matrices (W_o, dW) use the
 *    nn.Linear layout [out, in]; the activations X (local attention output)
 *    and Z (full attention output) are [tokens, hidden] with column
 *    head * head_dim + j, and the projection is Y = X W^T.
 *  - Device pointers must be 16-byte aligned (ISPA_ERR_ALIGN otherwise).
 *  - Calls on one stream execute in order; calls that write the same buffers
 *    from different streams must be ordered by the caller.
 */
#ifndef ISPA_H_
#define ISPA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ISPA_OK = 0,
  ISPA_ERR_NULL = 1,        /* a required pointer is NULL */
  ISPA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  ISPA_ERR_UNSUPPORTED = 3, /* a valid but unsupported configuration */
  ISPA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  ISPA_ERR_WORKSPACE = 5,   /* workspace missing or too small */
  ISPA_ERR_HIP = 6,         /* the HIP runtime reported an error (launch, copy, mapping) */
  ISPA_ERR_SCRATCH = 7      /* input too large for an allocation-free entry point's
                               fixed scratch */
};

/* Static text for a status code (never NULL). */
const char* ispa_status_string(int status);

/* Library version as major * 10000 + minor * 100 + patch. */
int ispa_version(void);

/*
 * Decomposable attention (§3.1 item 1 and §3.4).
 *
 * For each head and query row q of the chunk, with s_j = sm_scale * q . k_j:
 *   local   = softmax attention over the sink and current keys (A_loc),
 *   history = softmax attention over the history keys,
 *   full    = softmax attention over sink + history + current (A_full),
 * all from one pass over the KV: the local and history partial results are
 * merged through their log-sum-exp states. No mask inside the chunk.
 *
 * q                [n_q, n_heads, head_dim] bf16 (post-RoPE).
 * k_/v_sink        [n_sink, n_heads, head_dim] bf16; k_/v_cur [n_cur, ...];
 * k_/v_hist        [n_hist, ...]. Segments may live in separate buffers.
 * head_dim         64 or 128 (ISPA_ERR_UNSUPPORTED otherwise).
 * sm_scale         softmax scale (> 0, finite), normally 1/sqrt(head_dim).
 * Outputs (any may be NULL = not produced; at least one non-NULL):
 *   o_local, o_hist, o_full, d_out   [n_q, n_heads * head_dim] bf16,
 *   lse_local, lse_hist, lse_full    [n_heads, n_q] fp32, natural log.
 * d_out = O_full - O_local, formed in fp32 against the bf16-rounded O_local
 *   that o_local holds, so X + D tracks O_full as closely as bf16 allows.
 * An empty history (n_hist = 0) gives o_hist = 0, lse_hist = -inf,
 *   o_full = o_local and d_out = 0. n_sink + n_cur must be >= 1.
 * When only o_full / lse_full are requested the KV is traversed once
 *   without the split.
 * Errors: ISPA_ERR_NULL for a NULL q, a NULL segment pointer with a non-zero
 *   length, or no output; ISPA_ERR_SHAPE for negative sizes, n_heads < 1,
 *   n_sink + n_cur == 0 or a non-positive scale; ISPA_ERR_UNSUPPORTED for
 *   another head_dim.
 */
int ispa_attn_decomp(const void* q, int64_t n_q,
                     const void* k_sink, const void* v_sink, int64_t n_sink,
                     const void* k_cur, const void* v_cur, int64_t n_cur,
                     const void* k_hist, const void* v_hist, int64_t n_hist,
                     int n_heads, int head_dim, float sm_scale,
                     void* o_local, float* lse_local,
                     void* o_hist, float* lse_hist,
                     void* o_full, float* lse_full,
                     void* d_out, void* stream);

/*
 * The warmup step's attention with the statistics operands written
 * feature-major (§3.1 items 1-2: both signals from the one pass, then the
 * accumulated statistics over the tokens). Same inputs, arithmetic and
 * errors as ispa_attn_decomp; outputs:
 *   o_full            as in ispa_attn_decomp, required (ISPA_ERR_NULL);
 *   lse_full          as in ispa_attn_decomp, may be NULL;
 *   xt, dt            X = O_local and D = O_full - O_local, bf16, element
 *                     (query q, feature f = head * head_dim + j) at
 *                     [f * ld + q]: [n_heads * head_dim][ld], the same bf16
 *                     values ispa_attn_decomp writes to o_local and d_out.
 *                     Both required (ISPA_ERR_NULL). Columns >= n_q are not
 *                     touched, so the warmup steps of a layer can be written
 *                     side by side (xt + s * n_q with a common ld) and their
 *                     statistics formed in one ispa_gram_accumulate_t call.
 * ld >= n_q (ISPA_ERR_SHAPE), ld % 8 == 0 and xt, dt 16-byte aligned
 * (ISPA_ERR_ALIGN), n_heads * head_dim * ld * 2 < 2^31 bytes
 * (ISPA_ERR_UNSUPPORTED).
 */
int ispa_attn_decomp_t(const void* q, int64_t n_q,
                       const void* k_sink, const void* v_sink, int64_t n_sink,
                       const void* k_cur, const void* v_cur, int64_t n_cur,
                       const void* k_hist, const void* v_hist, int64_t n_hist,
                       int n_heads, int head_dim, float sm_scale,
                       void* o_full, float* lse_full, void* xt, void* dt, int64_t ld,
                       void* stream);

/*
 * Several attention calls in one launch (multi-instance batching: concurrent
 * streams, each with its own KV cache, as the paper's §3.3 instance-specific
 * state implies when several videos are generated at once). Each job is
 * one ispa_attn_decomp call with its own queries, KV segments, lengths and
 * outputs; n_heads, head_dim and sm_scale are shared. Every job is
 * validated as ispa_attn_decomp validates its arguments (the first failing
 * job's status is returned and nothing is launched); jobs with n_q = 0 are
 * skipped. 1 <= n_jobs <= ISPA_MAX_GROUP (ISPA_ERR_SHAPE otherwise). The
 * results are bit-identical to separate ispa_attn_decomp calls. Calls whose
 * own grid covers at least half the device's compute units run as launches
 * of their own; the others share one launch (the case grouping is for:
 * short chunks or few heads, each of which alone leaves most of the chip
 * idle).
 */
#define ISPA_MAX_GROUP 8
typedef struct {
  const void* q;
  int64_t n_q;
  const void* k_sink;
  const void* v_sink;
  int64_t n_sink;
  const void* k_cur;
  const void* v_cur;
  int64_t n_cur;
  const void* k_hist;
  const void* v_hist;
  int64_t n_hist;
  void* o_local;
  float* lse_local;
  void* o_hist;
  float* lse_hist;
  void* o_full;
  float* lse_full;
  void* d_out;
} ispa_attn_job;
int ispa_attn_decomp_grouped(const ispa_attn_job* jobs, int n_jobs, int n_heads, int head_dim,
                             float sm_scale, void* stream);

/*
 * Decomposable attention with E4M3 scores (§3.4 builds on FlashAttention-
 * style LSE states and cites SageAttention's 8-bit attention; §4.4 runs
 * ISPA with 8-bit quantization). Same arguments, outputs, split and merge
 * as ispa_attn_decomp, with the scores formed from OCP E4M3 codes:
 *   query row (token, head): scale s_q = absmax / 448, codes of q * (448 / absmax);
 *   keys: smoothed as k - mu (fp32), then per head and per run of 64 keys
 *     from each segment's start: s_k = absmax / 448, codes likewise;
 *   score = sm_scale * s_q * s_k * sum_c dq(q_c) dq(k_c), products exact,
 *     accumulated by the E4M3 matrix cores;
 *   every LSE output gets sm_scale * (q . mu) added back (fp32, from the
 *     bf16 q), so it estimates the unsmoothed LSE; the outputs O do not
 *     depend on mu (a per-query constant shift of the scores).
 * Codes round to nearest even; all-zero blocks get scale 0. V, P and P V
 * are as in ispa_attn_decomp.
 * k_mean           [n_heads, head_dim] bf16 smoothing vector mu, or NULL (mu = 0);
 *                  e.g. from ispa_key_mean.
 * head_dim         128 only (ISPA_ERR_UNSUPPORTED otherwise).
 * workspace        ispa_attn_fp8_workspace_bytes(n_q, n_sink, n_cur, n_hist,
 *                  n_heads, head_dim) bytes, 16-byte aligned: the codes and
 *                  scales (1 byte per Q/K element plus 4 bytes per scale).
 * Errors: those of ispa_attn_decomp, plus ISPA_ERR_WORKSPACE, and
 *   ISPA_ERR_SHAPE when a segment has more than 2^31 64-key tiles x heads.
 */
size_t ispa_attn_fp8_workspace_bytes(int64_t n_q, int64_t n_sink, int64_t n_cur,
                                     int64_t n_hist, int n_heads, int head_dim);
int ispa_attn_decomp_fp8(const void* q, int64_t n_q,
                         const void* k_sink, const void* v_sink, int64_t n_sink,
                         const void* k_cur, const void* v_cur, int64_t n_cur,
                         const void* k_hist, const void* v_hist, int64_t n_hist,
                         int n_heads, int head_dim, float sm_scale,
                         const void* k_mean,
                         void* o_local, float* lse_local,
                         void* o_hist, float* lse_hist,
                         void* o_full, float* lse_full,
                         void* d_out, void* workspace, size_t ws_bytes,
                         void* stream);

/*
 * Mean key of the given segments, per head and channel (the smoothing
 * vector of ispa_attn_decomp_fp8): mu [n_heads, head_dim] bf16 = the fp32
 * column sums over all n_sink + n_cur + n_hist keys (in a fixed order, so
 * the result is deterministic), divided by the count, rounded to bf16.
 * head_dim 128 only. workspace: ispa_key_mean_workspace_bytes(n_heads,
 * head_dim) bytes. Errors: ISPA_ERR_NULL, ISPA_ERR_SHAPE (no keys),
 * ISPA_ERR_UNSUPPORTED, ISPA_ERR_WORKSPACE, ISPA_ERR_ALIGN.
 */
size_t ispa_key_mean_workspace_bytes(int n_heads, int head_dim);
int ispa_key_mean(const void* k_sink, int64_t n_sink, const void* k_cur, int64_t n_cur,
                  const void* k_hist, int64_t n_hist, int n_heads, int head_dim,
                  void* mu, void* workspace, size_t ws_bytes, void* stream);

/*
 * Warmup statistics (§3.1 item 2: the accumulated dual-stream activations).
 *
 * For each of n_batch independent problems b (e.g. layers):
 *   G[b] (+)= X[b]^T X[b],  C[b] (+)= X[b]^T D[b],  E[b] (+)= D[b]^T D[b]
 * x, d   [n_batch][n_tok, h] bf16 (X = O_local, D = O_full - O_local).
 * G, C, E [n_batch][h, h] fp32; E may be NULL. On return G and E are full
 *   symmetric matrices. zero_first != 0 overwrites instead of adding.
 * Summation order is fixed: results are bitwise reproducible.
 * n_tok may be 0 (adds nothing, or zeroes with zero_first).
 * Errors: ISPA_ERR_NULL (x, d, G, C), ISPA_ERR_SHAPE (h < 1, n_tok < 0,
 *   n_batch < 1), ISPA_ERR_UNSUPPORTED (h not a multiple of 8).
 */
int ispa_gram_accumulate(const void* x, const void* d, int64_t n_tok, int h,
                         int n_batch, float* G, float* C, float* E,
                         int zero_first, void* stream);

/*
 * The warmup statistics from feature-major activations (the xt, dt of
 * ispa_attn_decomp_t): for each of n_batch problems b,
 *   G[b] (+)= X[b]^T X[b],  C[b] (+)= X[b]^T D[b],  E[b] (+)= D[b]^T D[b]
 * with token t of feature f at xt[b][f * ld + t], t < n_tok
 * (xt, dt: [n_batch][h][ld] bf16, batch stride h * ld). G, C, E as in
 * ispa_gram_accumulate (E may be NULL; G and E exactly symmetric; fixed
 * summation order). The contraction over tokens runs as a product of two
 * token-contiguous operands on 256 x 256 output tiles.
 * Errors: ISPA_ERR_NULL (xt, dt, G, C), ISPA_ERR_SHAPE (h < 1, n_tok < 0,
 *   n_batch < 1, ld < n_tok), ISPA_ERR_UNSUPPORTED (h % 8 != 0, or one
 *   layer's X^T of 2 GiB or more), ISPA_ERR_ALIGN (ld % 8 != 0 or a pointer
 *   not 16-byte aligned).
 */
int ispa_gram_accumulate_t(const void* xt, const void* dt, int64_t n_tok, int64_t ld, int h,
                           int n_batch, float* G, float* C, float* E, int zero_first,
                           void* stream);

/*
 * Closed-form absorb (§3.2, §4.1): for each layer l,
 *   dW = argmin ||X (W + dW) - Z W||_F^2 + lambda ||dW||_F^2
 *      = (G + lambda I)^{-1} C W        (W = Wo^T, math layout [in, out]),
 * computed as Y = (G + lambda I)^{-1} C by a blocked fp32 Cholesky
 * factorisation of G + lambda I and two triangular solves, then dW = Y W.
 * A layer whose fp32 solution may be off by more than 1e-4 relative in dW is
 * refined once: the residual C - (G + lambda I) Y accumulated in fp64, solved
 * with the same factor and added to Y. Which layers: the error of dW along 8
 * fixed pseudo-random directions, from the same fp64 residual and factor
 * applied to those directions only. Refined or not, dW is then within ~1e-4
 * of the fp64 solution of the given fp32 statistics up to
 * cond(G + lambda I) ~ 1e5 (rank-deficient statistics have
 * cond ~ ||G|| / lambda). lambda is added unscaled to the summed statistics.
 * G, C     [n_layers][h, h] fp32 (read only).
 * Wo       [n_layers][h, h] bf16, nn.Linear layout (read only).
 * dW       [n_layers][h, h] fp32 output, nn.Linear layout (like Wo).
 * info     [n_layers] int32 device output: 0 = solved; j > 0 = the leading
 *          minor of order j of G + lambda I is not positive definite (dW of
 *          that layer is then meaningless, but finite work was done).
 * workspace: device buffer of at least ispa_ridge_workspace_bytes(n_layers,
 *          h) bytes. After the call it holds C W (used by ispa_layer_score).
 * Errors: ISPA_ERR_NULL, ISPA_ERR_SHAPE (n_layers < 1, h < 1, lambda < 0 or
 *   not finite), ISPA_ERR_UNSUPPORTED (h not a multiple of 8),
 *   ISPA_ERR_WORKSPACE.
 */
size_t ispa_ridge_workspace_bytes(int n_layers, int h);
int ispa_ridge_solve(int n_layers, int h, const float* G, const float* C,
                     const void* Wo, float lambda, float* dW, int* info,
                     void* workspace, size_t ws_bytes, void* stream);

/*
 * Layer error and dynamic selection (§3.3). For each layer, over all warmup
 * tokens:
 *   eps_abs = ||X (W + dW) - Z W||_F^2
 *           = tr(W^T E W) - tr(dW^T C W) - lambda ||dW||_F^2  (at the ridge
 *             optimum, which the solve of ispa_ridge_solve reaches to ~1e-4
 *             relative or better), Z = X + D, clamped at 0 (a near-exact fit
 *             can come out below 0 by the fp32 rounding of the traces,
 *             ~2^-24 sqrt(h) of ||Z W||^2),
 *   eps_rel = eps_abs / ||Z W||_F^2, ||Z W||^2 = tr(W^T (G + C + C^T + E) W);
 *   eps_rel = 0 when both are 0, +inf when only the denominator is 0.
 * Layers with info != 0 or a NaN error get +inf and are never selected.
 * selected[l] = 1 for the min(K, #valid) layers with the lowest eps_rel
 *   (equal errors: lower layer index first), else 0.
 * workspace: the workspace of the ispa_ridge_solve call that produced dW, on
 *   the same stream and unchanged since (it reads C W from it and reuses the
 *   rest as scratch).
 * eps_abs, eps_rel [n_layers] fp64, selected [n_layers] int32: device outputs.
 * Errors: ISPA_ERR_NULL, ISPA_ERR_SHAPE (K < 0, ...), ISPA_ERR_WORKSPACE.
 */
int ispa_layer_score(int n_layers, int h, const float* G, const float* C,
                     const float* E, const void* Wo, const float* dW,
                     float lambda, const int* info, int K,
                     void* workspace, size_t ws_bytes,
                     double* eps_abs, double* eps_rel, int* selected,
                     void* stream);

/*
 * Weight injection (§3.3: W_new = W + dW, updated in place).
 * For every layer with selected[l] != 0 (device int32 [n_layers]):
 *   Wo[l] = bf16(Wo[l] + dW[l]), correctly rounded (nearest, ties to even)
 * from the exact sum. Other layers are untouched.
 * Wo [n_layers][h, h] bf16 in/out; dW [n_layers][h, h] fp32.
 * Errors: ISPA_ERR_NULL, ISPA_ERR_SHAPE, ISPA_ERR_UNSUPPORTED (h % 8 != 0).
 */
int ispa_apply_dW(int n_layers, int h, const int* selected, const float* dW,
                  void* Wo, void* stream);

/*
 * L-layer output projection (§3.1 item 3): y = x w^T.
 * x [n, h_in] bf16, w [h_out, h_in] bf16 (nn.Linear layout), y [n, h_out]
 * bf16 (fp32 accumulation, round to nearest even). No bias.
 * Errors: ISPA_ERR_NULL, ISPA_ERR_SHAPE, ISPA_ERR_UNSUPPORTED (h_in or h_out
 *   not a multiple of 8).
 */
int ispa_project(const void* x, const void* w, void* y, int64_t n, int h_in,
                 int h_out, void* stream);

/*
 * Several output projections in one launch (multi-instance batching: each
 * instance has its own W + dW, §3.3's instance-specific update): job g
 * computes y [n, h_out] = x [n, h_in] w^T as ispa_project does, with its
 * own x, w (bf16 [h_out, h_in]) and y; h_in and h_out are shared.
 * 1 <= n_jobs <= ISPA_MAX_GROUP and n >= 0 (ISPA_ERR_SHAPE);
 * h_in % 32 == 0, h_out % 8 == 0, and each x and w below 2^31 bytes
 * (ISPA_ERR_UNSUPPORTED); ISPA_ERR_NULL / ISPA_ERR_ALIGN for a job with
 * n > 0. Results are bit-identical to separate ispa_project calls.
 */
typedef struct {
  const void* x;
  const void* w;
  void* y;
  int64_t n;
} ispa_project_job;
int ispa_project_grouped(const ispa_project_job* jobs, int n_jobs, int h_in, int h_out,
                         void* stream);

/*
 * W8A8 output projection (§4.4, "Compatibility with Post-Training
 * Quantization": 8-bit weights and activations for the linear layers; for an
 * L-layer W + dW is quantized after ispa_apply_dW). Format: OCP 8-bit
 * floating point E4M3 ("fn": bias 7, no infinities, 0x7F / 0xFF NaN,
 * largest finite 448), one byte a code.
 *
 * ispa_quantize_fp8: per-row quantization of a [rows, k] bf16 matrix (k % 8
 *   == 0): scale[r] = absmax_r / 448 (fp32; 0 for an all-zero row) and
 *   q[r][c] = the E4M3 code nearest to fp32(a[r][c] * (448 / absmax_r)),
 *   ties to even (both divisions correctly rounded fp32). q [rows, k] uint8,
 *   scale [rows] fp32. For weights, rows are output channels.
 * ispa_project_w8a8: y [n, h_out] bf16 = X W^T with X = x [n, h_in] bf16
 *   quantized per token the same way (into the workspace) and W given as
 *   wq [h_out, h_in] E4M3 with w_scale [h_out]:
 *     y[m][o] = s_x[m] s_w[o] sum_k dq(Xq[m][k]) dq(Wq[o][k]),
 *   products exact, accumulated by the E4M3 matrix cores (their accumulation
 *   keeps ~1e-4 of the sum of |products| at worst), scaled, rounded to
 *   bf16. h_in % 64 == 0 and h_out % 8 == 0 (ISPA_ERR_UNSUPPORTED
 *   otherwise). workspace: ispa_project_w8a8_workspace_bytes(n, h_in).
 * Errors: ISPA_ERR_NULL, ISPA_ERR_SHAPE, ISPA_ERR_UNSUPPORTED,
 *   ISPA_ERR_WORKSPACE, ISPA_ERR_ALIGN.
 */
int ispa_quantize_fp8(const void* a, int64_t rows, int k, void* q, float* scale,
                      void* stream);
size_t ispa_project_w8a8_workspace_bytes(int64_t n, int h_in);
int ispa_project_w8a8(const void* x, const void* wq, const float* w_scale, void* y,
                      int64_t n, int h_in, int h_out, void* workspace,
                      size_t ws_bytes, void* stream);

/*
 * Allocation-free W8A8 projection, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): ispa_project_w8a8 without the workspace argument. The
 * quantized tokens are staged in a fixed scratch array of the library
 * (ISPA_NOALLOC_MAX_CODE_BYTES of codes plus ISPA_NOALLOC_MAX_TOKENS fp32
 * scales, 32.25 MiB), of which each GPU the library runs on holds its own
 * copy until the process ends. The call allocates nothing: on its first
 * call on a device (with that device current) it looks up that device's copy
 * with hipGetSymbolAddress, once. The caller passes inputs and outputs as
 * for ispa_project_w8a8 and gets the same result, bit for bit.
 * Calls on one GPU share its scratch: calls that overlap on one GPU (on
 * different streams, or from host threads without ordering between them)
 * race and must be serialised by the caller.
 * Errors: those of ispa_project_w8a8 (no ISPA_ERR_WORKSPACE), plus
 *   ISPA_ERR_SCRATCH when n > ISPA_NOALLOC_MAX_TOKENS or n * h_in >
 *   ISPA_NOALLOC_MAX_CODE_BYTES, and ISPA_ERR_HIP when the scratch address
 *   cannot be looked up.
 */
#define ISPA_NOALLOC_MAX_CODE_BYTES (32 * 1024 * 1024)
#define ISPA_NOALLOC_MAX_TOKENS 65536
int ispa_project_w8a8_noalloc(const void* x, const void* wq, const float* w_scale, void* y,
                              int64_t n, int h_in, int h_out, void* stream);

/*
 * Drift score for event-triggered recalibration (§3.3, last paragraph: on a
 * large scene transition or temporal distribution shift the warmup-to-
 * absorption procedure is re-entered; the pages give no trigger). For an
 * absorbed layer with warmup statistics G over N warmup tokens and
 * M = G + lambda I, the leverage of a token x (a row of the layer's local
 * output X) is x M^{-1} x^T, and its warmup expectation is
 * ref = tr(M^{-1} G) / N = (h - lambda tr(M^{-1})) / N. The score of a chunk
 * is the mean leverage of a strided sample of its tokens divided by ref:
 * about 1 while the activations stay in the span the update was fitted on,
 * large once they leave it (the absorbed dW then extrapolates).
 *
 * ispa_drift_prepare: for each layer, the lower Cholesky factor of M is
 *   inverted into linv ([n_layers][h, h] fp32, lower triangular, zeros
 *   above the diagonal) and ref [n_layers] fp64 is computed. info as for
 *   ispa_ridge_solve (linv and ref are meaningless where info != 0).
 *   workspace: ispa_ridge_workspace_bytes(n_layers, h) bytes at least.
 * ispa_drift_prepare_factored: the same linv and ref from the factor that the
 *   preceding ispa_ridge_solve(n_layers, h, G, ..., lambda, ...) left in its
 *   workspace, without factoring M again. The workspace must be that call's,
 *   on the same stream, with no ispa_layer_score (which reuses the factor's
 *   storage) or other call on it in between; the failure flags are that
 *   call's info. Bit-identical to ispa_drift_prepare on the same G and lambda.
 * ispa_drift_score: x [n_layers][n_tok, h] bf16; the sample is the rows
 *   0, stride, 2 stride, ... (ceil(n_tok / stride) of them); score
 *   [n_layers] fp64 out (+inf when ref is 0); ref and score need only
 *   8-byte alignment (one layer's entry may be passed alone). workspace:
 *   ispa_drift_workspace_bytes(n_layers, h, ceil(n_tok / stride)) bytes.
 * ispa_drift_workspace_bytes covers both calls (0 for invalid sizes).
 * Errors: ISPA_ERR_NULL, ISPA_ERR_SHAPE (sizes < 1, lambda < 0 or not
 *   finite), ISPA_ERR_UNSUPPORTED (h % 8 != 0), ISPA_ERR_WORKSPACE,
 *   ISPA_ERR_ALIGN.
 */
size_t ispa_drift_workspace_bytes(int n_layers, int h, int64_t n_sample);
int ispa_drift_prepare(int n_layers, int h, const float* G, float lambda,
                       int64_t n_warm, float* linv, double* ref, int* info,
                       void* workspace, size_t ws_bytes, void* stream);
int ispa_drift_prepare_factored(int n_layers, int h, float lambda, int64_t n_warm,
                                float* linv, double* ref, void* workspace, size_t ws_bytes,
                                void* stream);
int ispa_drift_score(int n_layers, int h, const float* linv, const double* ref,
                     const void* x, int64_t n_tok, int64_t stride, double* score,
                     void* workspace, size_t ws_bytes, void* stream);

/*
 * ------------------------------------------------------------------------
 * Streaming KV cache and the per-layer streaming step (§3.1 item 3 and
 * §3.3: after the transition the K selected layers (L-layers) attend the
 * sink and current tokens only, through W + dW, and drop their history KV
 * for good; the other layers (F-layers) keep attending their whole history
 * through W).
 *
 * One cache holds, for each of n_layers layers, the K and V rows
 * ([n_heads, head_dim] bf16 each) of the sink (n_sink tokens, written once),
 * of the current chunk (n_cur tokens, written every chunk) and of the
 * history. Each layer's K and V live in one reserved virtual address range
 * laid out as [sink | slot 0 | ... | slot S-1], one chunk per slot,
 * S = hist_capacity / n_cur + 1: chunk c of an F-layer sits in slot c mod S
 * and its history is every other filled slot, i.e. the min(c, S - 1) most
 * recent chunks (a capacity at least as long as the stream keeps all of it).
 * Physical memory is mapped page by page as slots are first used (a page
 * is the smallest power of two holding one chunk, 2 MiB to 256 MiB) and
 * released when a layer turns local-only, so resident memory follows the
 * history that is actually kept, to within one page per layer and tensor. The chunk's K/V are written in place (into the pointers of
 * ispa_kv_view_of, or with ispa_kv_write) and never move.
 *
 * Life cycle per chunk: write each layer's current K/V; run the layers
 * (ispa_kv_attn / ispa_kv_layer_forward); then ispa_kv_advance once, which
 * makes the chunk part of every F-layer's history. ispa_kv_evict_history
 * turns a layer into an L-layer between chunks (after ispa_kv_advance and
 * before the next chunk's K/V are written).
 *
 * The cache is host-side state: its calls are not thread-safe on one cache.
 * ispa_kv_create, ispa_kv_advance, ispa_kv_evict_history and
 * ispa_kv_destroy allocate or free device memory (HIP virtual memory
 * management); the other calls only enqueue work like the calls above.
 * ------------------------------------------------------------------------
 */
typedef struct ispa_kv_cache ispa_kv_cache;

enum { ISPA_KV_CURRENT = 0, ISPA_KV_SINK = 1 };

/* Where one layer's rows are, for the chunk that is current. */
typedef struct ispa_kv_view {
  void* k_sink; void* v_sink;   /* n_sink rows */
  void* k_cur;  void* v_cur;    /* n_cur rows of the current chunk */
  /* The three KV segments ispa_attn_decomp takes, in its order. When
   * split_ok != 0 they are exactly (sink, current, history); otherwise (an
   * F-layer whose ring has wrapped) their union is sink + history + current
   * and only the full outputs of ispa_attn_decomp over them are meaningful
   * (ispa_kv_attn forms the split outputs in that case too). A segment of
   * length 0 has NULL pointers. */
  const void* seg_k[3];
  const void* seg_v[3];
  int64_t seg_n[3];
  int64_t n_hist;               /* history tokens */
  int32_t split_ok;
  int32_t local_only;           /* 1 after ispa_kv_evict_history */
} ispa_kv_view;

/*
 * Create a cache on the current device. head_dim is 64 or 128;
 * hist_capacity (tokens) must be a multiple of n_cur. Maps the sink and the
 * first slot of every layer. *out is a host handle (NULL on error).
 * Errors: ISPA_ERR_NULL (out), ISPA_ERR_SHAPE (n_layers, n_heads, n_cur < 1,
 *   n_sink or hist_capacity < 0, hist_capacity % n_cur != 0, sizes that
 *   overflow), ISPA_ERR_UNSUPPORTED (head_dim; device without virtual
 *   memory management), ISPA_ERR_HIP (reservation or mapping failed, e.g.
 *   out of device memory).
 */
int ispa_kv_create(int n_layers, int n_heads, int head_dim, int64_t n_sink,
                   int64_t n_cur, int64_t hist_capacity, ispa_kv_cache** out);

/* Waits for the device, then frees every range. ISPA_ERR_NULL for NULL. */
int ispa_kv_destroy(ispa_kv_cache* cache);

/* Host-side copy of layer `layer`'s view. Errors: ISPA_ERR_NULL,
 * ISPA_ERR_SHAPE (layer out of range). */
int ispa_kv_view_of(const ispa_kv_cache* cache, int layer, ispa_kv_view* view);

/*
 * Copy rows into the layer's current slot (which = ISPA_KV_CURRENT, n_cur
 * rows) or sink (ISPA_KV_SINK, n_sink rows), device to device, on `stream`.
 * k, v: [rows, n_heads, head_dim] bf16.
 * Errors: ISPA_ERR_NULL, ISPA_ERR_SHAPE (layer, which), ISPA_ERR_HIP.
 */
int ispa_kv_write(ispa_kv_cache* cache, int layer, int which, const void* k,
                  const void* v, void* stream);

/*
 * End of a chunk: every F-layer's current chunk joins its history and the
 * next slot is mapped (the oldest chunk is dropped once the ring is full).
 * L-layers keep writing slot 0. Host call; enqueues nothing. On
 * ISPA_ERR_HIP (mapping failed) no layer has moved.
 */
int ispa_kv_advance(ispa_kv_cache* cache);

/*
 * Turn a layer into an L-layer: waits for `stream` (work on other streams
 * that reads the layer must be complete), then unmaps and frees its history;
 * the sink and slot 0 stay. Idempotent. Errors: ISPA_ERR_NULL,
 * ISPA_ERR_SHAPE, ISPA_ERR_HIP.
 */
int ispa_kv_evict_history(ispa_kv_cache* cache, int layer, void* stream);

/* Text of the last failed HIP call made by the cache's management calls
 * (which call, offset and size within the layer's range, HIP's message), or
 * "" if none failed. With cache = NULL: the last failed ispa_kv_create on
 * the calling thread. The text lives as long as the cache (or the thread). */
const char* ispa_kv_last_error(const ispa_kv_cache* cache);

/*
 * Turn an L-layer back into a full-history layer for a recalibration
 * (§3.3, last paragraph): its history restarts empty with the current chunk
 * (slot 0), and grows again from the next ispa_kv_advance. Call between
 * chunks, like ispa_kv_evict_history. No effect on a full-history layer.
 * Errors: ISPA_ERR_NULL, ISPA_ERR_SHAPE.
 */
int ispa_kv_restore_history(ispa_kv_cache* cache, int layer);

/* Device bytes currently mapped for K and V of all layers (-1 for NULL). */
int64_t ispa_kv_resident_bytes(const ispa_kv_cache* cache);

/*
 * ispa_attn_decomp of one layer over its cache for the current chunk:
 * q [n_q, n_heads, head_dim] bf16, outputs as there. For an F-layer whose
 * ring has wrapped (split_ok == 0) the split outputs are formed over its
 * history in the ring's two pieces (slots after the current one, then the
 * slots before it). For an L-layer the history is empty. Errors as for
 * ispa_attn_decomp, plus ISPA_ERR_SHAPE for the layer index.
 */
int ispa_kv_attn(const ispa_kv_cache* cache, int layer, const void* q,
                 int64_t n_q, float sm_scale, void* o_local, float* lse_local,
                 void* o_hist, float* lse_hist, void* o_full, float* lse_full,
                 void* d_out, void* stream);

/*
 * One layer's attention and output projection in the stream: an L-layer
 * computes O = local attention, an F-layer O = full attention (one pass),
 * into o_tmp [n_q, h] bf16, then y = O wo^T ([n_q, h] bf16, h = n_heads *
 * head_dim, wo [h, h] bf16 in nn.Linear layout: W + dW for an L-layer after
 * ispa_apply_dW, W for an F-layer). Errors as ispa_kv_attn and ispa_project;
 * nothing is enqueued on error.
 */
int ispa_kv_layer_forward(const ispa_kv_cache* cache, int layer, const void* q,
                          int64_t n_q, float sm_scale, const void* wo,
                          void* o_tmp, void* y, void* stream);

/*
 * ------------------------------------------------------------------------
 * Streaming session: the warmup -> absorption -> streaming life cycle of all
 * attention layers over one KV cache (§3.1 items 1-3, §3.3), with
 * event-triggered recalibration (§3.3, last paragraph) driven by the drift
 * score above. Host-side control; every step is one of the calls above,
 * enqueued on the caller's stream.
 *
 * Per chunk: write every layer's current K/V (ispa_session_cache +
 * ispa_kv_view_of / ispa_kv_write; the sink once, before the first chunk),
 * run ispa_session_layer for each layer in order, then
 * ispa_session_end_chunk once. The queries of a chunk are its n_cur tokens.
 *  - warmup phase (from creation, and after a recalibration): every layer
 *    runs the dual-stream attention, accumulates G, C, E over the phase's
 *    chunks (statistics start over with each warmup) and outputs
 *    y = O_full W^T with the original W. After t_warm chunks, end_chunk
 *    solves dW against the original W, scores, selects k_select layers,
 *    writes bf16(W + dW) for them into w_active, drops their history and
 *    (drift_threshold > 0) prepares their drift state: event ABSORBED.
 *  - stream phase: L-layers y = O_local (W + dW)^T, F-layers
 *    y = O_full W^T; each L-layer's O_local gets a drift score (sample
 *    stride drift_stride). If one exceeds drift_threshold (or is NaN),
 *    end_chunk restores the L-layers (original W, history restarting with
 *    the next chunk) and enters warmup again: event RECALIBRATE.
 * A warmup after a recalibration attends each F-layer's history as the
 * cache holds it: the hist_capacity most recent tokens, also once the ring
 * has wrapped.
 *
 * Memory: wo [n_layers][h, h] bf16 (original weights, read, kept unchanged
 * by the caller), w_active [n_layers][h, h] bf16 (written: the weights in
 * use), workspace of ispa_session_workspace_bytes bytes (statistics, dW,
 * drift factors, solver scratch, one chunk of activations); the session's
 * KV cache allocates its own pages. end_chunk synchronises `stream` at the
 * transition and, with recalibration on, at every streaming chunk (it reads
 * the selection and the drift scores on the host).
 * ------------------------------------------------------------------------
 */
typedef struct ispa_session ispa_session;

enum { ISPA_PHASE_WARMUP = 0, ISPA_PHASE_STREAM = 1 };
enum { ISPA_EVENT_NONE = 0, ISPA_EVENT_ABSORBED = 1, ISPA_EVENT_RECALIBRATE = 2 };

/* Session flags (the quantized variant, §4.4 and §3.4's cited 8-bit
 * attention):
 *  ISPA_SESSION_W8A8      every output projection runs as ispa_project_w8a8
 *                         on E4M3 weights with one scale per output channel,
 *                         quantized from the active bf16 weights whenever they
 *                         change (creation, absorption, recalibration), so an
 *                         L-layer's W + dW is folded in before quantization;
 *                         needs n_heads * head_dim % 64 == 0.
 *  ISPA_SESSION_FP8_ATTN  the streaming phase's attention runs as
 *                         ispa_attn_decomp_fp8, smoothed by the layer's mean
 *                         sink key (the current chunk's keys when n_sink is
 *                         0), fixed at the layer's first streamed chunk; the
 *                         warmup keeps bf16 attention for the statistics.
 *                         head_dim 128 only. */
enum { ISPA_SESSION_W8A8 = 1, ISPA_SESSION_FP8_ATTN = 2 };

typedef struct ispa_session_config {
  int32_t n_layers, n_heads, head_dim;   /* head_dim 64 or 128 */
  int32_t k_select;                      /* layers absorbed per transition */
  int32_t t_warm;                        /* warmup chunks per calibration (>= 1) */
  int32_t flags;                         /* ISPA_SESSION_* bits, 0 = bf16 throughout */
  int64_t n_sink, n_cur, hist_capacity;  /* tokens; hist_capacity % n_cur == 0 */
  float sm_scale, lambda;
  double drift_threshold;                /* <= 0: never recalibrate */
  int64_t drift_stride;                  /* >= 1 */
} ispa_session_config;

typedef struct ispa_session_state {
  int32_t phase, warm_count, n_calibrations, reserved;
  int64_t chunk;                         /* chunks ended so far */
} ispa_session_state;

/* Workspace bytes for a configuration (0 if it is invalid). */
size_t ispa_session_workspace_bytes(const ispa_session_config* cfg);

/* Create a session (and its KV cache) on the current device; copies wo into
 * w_active on `stream` (and, with ISPA_SESSION_W8A8, quantizes it).
 * Errors: ISPA_ERR_NULL, ISPA_ERR_SHAPE (invalid configuration or unknown
 * flag bits), ISPA_ERR_UNSUPPORTED (head_dim, or a flag the shape does not
 * allow), ISPA_ERR_WORKSPACE, ISPA_ERR_ALIGN, and those of ispa_kv_create. */
int ispa_session_create(const ispa_session_config* cfg, const void* wo,
                        void* w_active, void* workspace, size_t ws_bytes,
                        void* stream, ispa_session** out);
int ispa_session_destroy(ispa_session* s);
/* The session's KV cache, to write the chunks' K/V (NULL for NULL). */
ispa_kv_cache* ispa_session_cache(ispa_session* s);
/* One layer of the current chunk: q [n_cur, n_heads, head_dim] bf16,
 * y [n_cur, h] bf16 out. Errors of the calls it makes. */
int ispa_session_layer(ispa_session* s, int layer, const void* q, void* y,
                       void* stream);
/* The same layer of n concurrent sessions (multi-instance batching), with
 * the same results as n ispa_session_layer calls: the streaming-phase
 * sessions without flags run their attention as one grouped launch and
 * their projections (each through its own active weights) as another; the
 * others run one by one. The sessions must share n_heads, head_dim and
 * n_cur (ISPA_ERR_SHAPE otherwise); 1 <= n <= ISPA_MAX_GROUP. */
int ispa_session_layer_grouped(ispa_session* const* s, int n, int layer,
                               const void* const* q, void* const* y, void* stream);
/* End of a chunk; *event (may be NULL) receives ISPA_EVENT_*. */
int ispa_session_end_chunk(ispa_session* s, void* stream, int* event);
/* Phase and counters; with non-NULL host arrays of n_layers entries also
 * the current L-layer mask, the errors of the last transition and the last
 * drift scores (0 for F-layers). */
int ispa_session_query(const ispa_session* s, ispa_session_state* out,
                       int* is_local, double* eps_rel, double* drift);

#ifdef __cplusplus
}
#endif

#endif /* ISPA_H_ */
