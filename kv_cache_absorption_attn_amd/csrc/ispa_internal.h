// Internal launch interface between the C-ABI entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ispa {

// ---------------------------------------------------------------- attention
struct AttnParams {
  const uint16_t* q;         // [n_q, n_heads, D] bf16
  // segments: 0 sink and 1 current (the local set), 2 and 3 history (one
  // piece, or the two pieces of a ring buffer that has wrapped; n[3] = 0
  // otherwise)
  const uint16_t* k[4];
  const uint16_t* v[4];
  int64_t n[4];
  int64_t n_q;
  int n_heads;
  float scale_log2;          // softmax scale * log2(e)
  uint16_t* o_local;         // [n_q, n_heads*D] bf16 (any may be null)
  float* lse_local;          // [n_heads, n_q]
  uint16_t* o_hist;
  float* lse_hist;
  uint16_t* o_full;
  float* lse_full;
  uint16_t* d_out;
  // feature-major copies of X = O_local and of D (element (query q, feature
  // f) at [f * ldt + q]), the operands of the feature-major Gram; either may
  // be null, and they are written only when a token-major output holds the
  // parked X (o_local, o_full or d_out)
  uint16_t* xt;
  uint16_t* dt;
  int64_t ldt;
  int n_qtiles;
  int mode;                  // 0: local / history split + merge; 1: one pass (full only)
  int need_hist;             // split mode: history phase and merge needed
  // E4M3 scores (head_dim 128; used when q8 is set): query codes [n_q,
  // n_heads, D] with scales [n_heads, n_q]; per segment the smoothed key
  // codes [n_s, n_heads, D] with scales [tiles_s, n_heads] (64-key tiles);
  // qmu [n_heads, n_q]: scale * q . mu added to every LSE output (or null)
  const uint8_t* q8;
  const float* qsc;
  const uint8_t* k8[4];
  const float* ksc[4];
  const float* qmu;
};
// Fills p.n_qtiles, then launches.
hipError_t launch_attn_decomp(AttnParams p, int head_dim, hipStream_t stream);
// Up to kMaxGroup calls with the same head_dim and precision in one launch
// (the table travels as the kernel argument); fills n_qtiles and start.
constexpr int kMaxGroup = 8;
struct AttnGroup {
  AttnParams p[kMaxGroup];
  int start[kMaxGroup + 1];
  int n;
};
hipError_t launch_attn_grouped(AttnGroup grp, int head_dim, hipStream_t stream);

// ispa_attn_decomp with the history in two pieces (hist, then hist2: the two
// ranges of a ring buffer that has wrapped): the same arguments, checks,
// outputs and errors; the second piece may be empty.
int attn_decomp_two_piece_history(const void* q, int64_t n_q, const void* k_sink,
                                  const void* v_sink, int64_t n_sink, const void* k_cur,
                                  const void* v_cur, int64_t n_cur, const void* k_hist,
                                  const void* v_hist, int64_t n_hist, const void* k_hist2,
                                  const void* v_hist2, int64_t n_hist2, int n_heads, int head_dim,
                                  float sm_scale, void* o_local, float* lse_local, void* o_hist,
                                  float* lse_hist, void* o_full, float* lse_full, void* d_out,
                                  void* stream);

// E4M3 attention operands (head_dim 128).
struct KeySegs {
  const uint16_t* k[3];      // [n_s, n_heads, 128] bf16
  int64_t n[3];
};
hipError_t launch_quantize_queries_fp8(const uint16_t* q, int64_t n_q, int n_heads,
                                       const uint16_t* mu, float sm_scale, uint8_t* q8,
                                       float* qsc, float* qmu, hipStream_t stream);
int64_t key_tiles(int64_t n);  // 64-key tiles of a segment
hipError_t launch_quantize_key_tiles_fp8(const uint16_t* k, int64_t n, int n_heads,
                                         const uint16_t* mu, uint8_t* k8, float* ksc,
                                         hipStream_t stream);
int key_mean_splits();         // partial sums of the key mean (rows of its workspace)
hipError_t launch_key_mean(const KeySegs& segs, int n_heads, float* part, uint16_t* mu,
                           hipStream_t stream);
int attn_q_tile_min();  // smallest query tile of any attention kernel

// ---------------------------------------------------------------- Gram
struct GramParams {
  const uint16_t* x;         // [batch][n_tok, h] bf16
  const uint16_t* d;         // null: G only
  int64_t n_tok;
  int h;
  int batch;
  float* G;                  // [batch][h, h] fp32
  float* C;
  float* E;                  // may be null
  int zero_first;
};
hipError_t launch_gram(const GramParams& p, hipStream_t stream);
// Y[b] = C[b] W[b]^T-style product in fp32: Y[b][i][o] = sum_k C[b][i][k] W[b][o][k]
// for fp32 C (split into two bf16 planes hi, lo of [batch][h, h] each) and
// bf16 W; bf16 matrix cores, fp32 accumulate.
hipError_t launch_split_nt_gemm_f32(const float* c, uint16_t* hi, uint16_t* lo,
                                    const uint16_t* w, float* y, int h, int batch,
                                    hipStream_t stream);

// ---------------------------------------------------------------- fp32 GEMM
// C[b](m, n) = alpha * sum_k A[b](m, k) B[b](k, n) + beta * C[b](m, n)
// Operand element (i, j) lives at ptr[i * s0 + j * s1]; one of the two
// strides of A and of B must be 1 (that dimension is loaded contiguously).
// C is row-major with leading dimension ldc. A may be bf16 (a_bf16 = 1).
struct GemmF32Params {
  int M, N, K;
  const void* A;
  int64_t a_s0, a_s1, a_batch;
  int a_bf16;
  const void* B;
  int64_t b_s0, b_s1, b_batch;
  int b_bf16;
  float* Cm;
  int64_t ldc, c_batch;
  float alpha, beta;
  int batch;
  int tri;                   // 0 all tiles; 1 only tiles with tile_m >= tile_n
  const int* layer_mask;     // optional [batch]: entries with mask 0 are skipped
};
hipError_t launch_gemm_f32(const GemmF32Params& p, hipStream_t stream);

// S[b] = C[b] - lam Y[b] - G[b] Y[b] for h x h fp32 row-major matrices, the
// products and the sum in fp64 (the residual of one refinement step).
struct RidgeResidParams {
  int h, batch;
  const float* G;
  const float* C;
  const float* Y;
  float* S;
  double lam;
  const int* layer_mask;     // optional [batch]: entries with mask 0 are skipped
};
hipError_t launch_ridge_resid_f64(const RidgeResidParams& p, hipStream_t stream);
// y[b][i] += x[b][i] over batch blocks of n fp32 elements each (n % 4 == 0,
// 16-byte aligned); blocks whose layer_mask entry is 0 are skipped (no mask:
// all of them).
hipError_t launch_add_inplace(float* y, const float* x, int64_t n, int batch,
                              const int* layer_mask, hipStream_t stream);

// Probe estimate of the refinement's need (see ispa_ridge_solve). For each
// layer b of an h x h problem with 8 probe columns:
//   launch_probe_wz:  Q[b] = W[b] Z, W(k, o) = Wo[b][o][k] (bf16, nn.Linear
//                     layout), Z[o][j] = +-1 from a fixed hash of (o, j);
//                     Q fp64 [h][8].
//   launch_mv8_f64:   Y[b] = X[b] Q[b] with X fp32 [h][h] row-major, Q and Y
//                     fp64 [h][8], accumulated in fp64.
//   launch_probe_resid: R[b] = A[b] - T[b] - lam B[b], written as fp32 [h][8].
//   launch_probe_flag: flag[b] = 1 unless ||E[b]||_F <= tol ||B[b]||_F (fp64
//                     sums in a fixed order; NaN flags 1).
hipError_t launch_probe_wz(const uint16_t* Wo, double* Q, int h, int batch, hipStream_t stream);
hipError_t launch_mv8_f64(const float* X, const double* Q, double* Y, int h, int batch,
                          hipStream_t stream);
hipError_t launch_probe_resid(const double* A, const double* T, const double* B, double lam,
                              float* R, int h, int batch, hipStream_t stream);
hipError_t launch_probe_flag(const float* E, const double* B, double tol, int* flag, int h,
                             int batch, hipStream_t stream);

// ---------------------------------------------------------------- ridge pieces
hipError_t launch_copy_add_diag(const float* G, float* L, int h, int batch, float lam,
                                hipStream_t stream);
// Diagonal block [k0, k0+nb) of L (nb <= 128): factor in place, write its
// inverse to Linv + k0 * 128 ([nb][128] row-major), record failures in info.
hipError_t launch_potrf_block(float* L, float* Linv, int h, int k0, int nb, int batch,
                              int* info, int info_first, hipStream_t stream);
// dst[b] = src[b]^T for h x h fp32 matrices.
hipError_t launch_transpose(const float* src, float* dst, int h, int batch, hipStream_t stream);
constexpr int kCholBlock = 128;

// ---------------------------------------------------------------- score / select / apply
struct ScoreParams {
  int n_layers, h;
  const float* G;
  const float* C;
  const float* E;
  const uint16_t* Wo;        // [L][out, in] bf16
  const float* dW;           // [L][out, in] fp32
  float lam;
  const int* info;
  int K;
  double* partial;           // workspace for per-tile partial sums
  double* eps_abs;
  double* eps_rel;
  int* selected;
};
// P = W W^T (lower 128-tiles valid), Bt = (C W)^T in nn.Linear layout.
hipError_t launch_score(const ScoreParams& p, const float* P, const float* Bt,
                        hipStream_t stream);
size_t layer_score_partial_count(int n_layers, int h);

hipError_t launch_apply_dw(int n_layers, int h, const int* selected, const float* dW,
                           uint16_t* Wo, hipStream_t stream);

// ---------------------------------------------------------------- drift score
hipError_t launch_identity(float* M, int h, int batch, hipStream_t stream);
// Row blocks of the summed-squares reduction of a matrix with `rows` rows.
int drift_partial_count(int rows);
// Summed squares S of each rows x cols fp32 matrix A[b] (row stride ld,
// matrix stride mat_stride), then out[b] = (h - lam S) / n_div when ref is
// null, else (S / n_div) / ref[b]. partial: batch * drift_partial_count(rows).
hipError_t launch_drift_sum(const float* A, int rows, int cols, int64_t ld, int64_t mat_stride,
                            int batch, double* partial, double h, double lam, double n_div,
                            const double* ref, double* out, hipStream_t stream);

// ---------------------------------------------------------------- projection
// The 256 x 128-tile NT GEMM (contraction length a multiple of 32).
bool nt_gemm256_supported(int h_in);
hipError_t launch_nt_gemm256_bf16(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t n,
                                  int h_in, int h_out, hipStream_t stream);
// E4M3 operands (contraction length a multiple of 64), scales per row of X
// and per row of W, bf16 out.
bool nt_gemm256_fp8_supported(int h_in);
// Up to kMaxGroup bf16 products Y_g = X_g W_g^T with shared h_in (% 32 == 0)
// and h_out in one launch; each X_g and W below 2^31 bytes.
struct NtJob {
  const uint16_t* x;
  const uint16_t* w;
  uint16_t* y;
  int64_t n;
};
hipError_t launch_nt_gemm256_grouped(const NtJob* jobs, int n_jobs, int h_in, int h_out,
                                     hipStream_t stream);
hipError_t launch_nt_gemm256_fp8(const uint8_t* xq, const float* sx, const uint8_t* wq,
                                 const float* sw, uint16_t* y, int64_t n, int h_in, int h_out,
                                 hipStream_t stream);
// Per-row E4M3 quantization of a bf16 [rows, k] matrix (k % 8 == 0).
hipError_t launch_quantize_rows_fp8(const uint16_t* a, int64_t rows, int k, uint8_t* q,
                                    float* scale, hipStream_t stream);
hipError_t launch_nt_gemm256_split_f32(const uint16_t* hi, const uint16_t* lo, const uint16_t* w,
                                       float* y, int h, int batch, hipStream_t stream);
hipError_t launch_project(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t n,
                          int h_in, int h_out, hipStream_t stream);

// The 256 x 256-tile NT GEMM (gemm256.hip).
// Y = X W^T, bf16 out; contraction length a multiple of 8 (any length works;
// the last stage is masked). row_tile 256 or 192: the tile height (the rows
// of X a workgroup covers; 192-row tiles fit more row counts into whole
// rounds of the chip).
hipError_t launch_g256_bf16(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t n,
                            int h_in, int h_out, hipStream_t stream, int row_tile = 256);
// Y[b] = (hi[b] + lo[b]) W[b]^T in fp32 for h x h operands (an fp32 matrix
// held as two bf16 planes times a bf16 matrix).
hipError_t launch_g256_split_f32(const uint16_t* hi, const uint16_t* lo, const uint16_t* w,
                                 float* y, int h, int batch, hipStream_t stream);
// Warmup statistics from feature-major activations: X^T, D^T [batch][h][ld]
// bf16 (token t of feature f at f * ld + t, n_tok <= ld, ld % 8 == 0):
// G = X^T X, C = X^T D, E = D^T D (fp32 [batch][h][h]; E may be null),
// accumulated or overwritten (zero_first); G and E exactly symmetric.
hipError_t launch_gram_t(const uint16_t* xt, const uint16_t* dt, int64_t n_tok, int64_t ld, int h,
                         int batch, float* G, float* C, float* E, int zero_first,
                         hipStream_t stream);

}  // namespace ispa
