// C ABI of the ISPA hot path: argument validation, workspace layout and the
// launch sequence of each entry point. Declarations and contracts are in
// include/ispa.h.

#include <math.h>
#include <stdint.h>

#include "ispa.h"
#include "ispa_internal.h"

namespace {

using ispa::kCholBlock;

// Relative error of dW0 = Y0 W (the fp32 solve) above which a layer's solve
// is refined: a tenth of the 1e-3 to which dW is held.
constexpr double kRefineTol = 1e-4;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

int hip_status(hipError_t e) { return e == hipSuccess ? ISPA_OK : ISPA_ERR_HIP; }

#define ISPA_TRY(expr)                       \
  do {                                       \
    const hipError_t e_ = (expr);            \
    if (e_ != hipSuccess) return ISPA_ERR_HIP; \
  } while (0)

size_t align_up(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

struct RidgeWs {
  float* L;       // [n_layers][h, h] Cholesky factor (later: W W^T for scoring)
  float* R;       // [n_layers][h, h] right-hand side -> (G + lambda I)^-1 C
  float* S;       // [n_layers][h, h] refinement residual / correction, staging
  float* Bt;      // [n_layers][h, h] (C W)^T in nn.Linear layout
  float* Linv;    // [n_layers][h, 128] inverses of the diagonal blocks
  double* part;   // layer-score partial sums
  int* refine;    // [n_layers] 1 where the solve is refined
  double* pq;     // [n_layers][h, 8] probe columns W z (the refinement estimate)
  double* pa;     // [n_layers][h, 8] C W z
  double* pb;     // [n_layers][h, 8] Y0 W z
  double* pt;     // [n_layers][h, 8] G Y0 W z
  float* pe;      // [n_layers][h, 8] residual, then the error estimate
  size_t bytes;
};

RidgeWs ridge_layout(void* base, int n_layers, int h) {
  RidgeWs w{};
  const size_t hh = static_cast<size_t>(h) * h * n_layers * sizeof(float);
  const size_t lin = static_cast<size_t>(h) * kCholBlock * n_layers * sizeof(float);
  const size_t part = ispa::layer_score_partial_count(n_layers, h) * sizeof(double);
  char* p = static_cast<char*>(base);
  size_t off = 0;
  w.L = reinterpret_cast<float*>(p + off);    off = align_up(off + hh);
  w.R = reinterpret_cast<float*>(p + off);    off = align_up(off + hh);
  w.S = reinterpret_cast<float*>(p + off);    off = align_up(off + hh);
  w.Bt = reinterpret_cast<float*>(p + off);   off = align_up(off + hh);
  w.Linv = reinterpret_cast<float*>(p + off); off = align_up(off + lin);
  w.part = reinterpret_cast<double*>(p + off); off = align_up(off + part);
  w.refine = reinterpret_cast<int*>(p + off);  off = align_up(off + n_layers * sizeof(int));
  const size_t probe = static_cast<size_t>(h) * 8 * n_layers;
  w.pq = reinterpret_cast<double*>(p + off); off = align_up(off + probe * sizeof(double));
  w.pa = reinterpret_cast<double*>(p + off); off = align_up(off + probe * sizeof(double));
  w.pb = reinterpret_cast<double*>(p + off); off = align_up(off + probe * sizeof(double));
  w.pt = reinterpret_cast<double*>(p + off); off = align_up(off + probe * sizeof(double));
  w.pe = reinterpret_cast<float*>(p + off);  off = align_up(off + probe * sizeof(float));
  w.bytes = off;
  return w;
}

// One fp32 GEMM over all layers: operand (i, j) at ptr[i * s0 + j * s1].
hipError_t gemm(int M, int N, int K, const void* A, int64_t a_s0, int64_t a_s1, int64_t a_batch,
                bool a_bf16, const void* B, int64_t b_s0, int64_t b_s1, int64_t b_batch,
                bool b_bf16, float* C, int64_t ldc, int64_t c_batch, float alpha, float beta,
                int batch, bool tri, hipStream_t s, const int* mask = nullptr) {
  ispa::GemmF32Params p{};
  p.M = M; p.N = N; p.K = K;
  p.A = A; p.a_s0 = a_s0; p.a_s1 = a_s1; p.a_batch = a_batch; p.a_bf16 = a_bf16;
  p.B = B; p.b_s0 = b_s0; p.b_s1 = b_s1; p.b_batch = b_batch; p.b_bf16 = b_bf16;
  p.Cm = C; p.ldc = ldc; p.c_batch = c_batch;
  p.alpha = alpha; p.beta = beta; p.batch = batch; p.tri = tri ? 1 : 0;
  p.layer_mask = mask;
  return ispa::launch_gemm_f32(p, s);
}

// Block rows [ba, bb) of R (128 rows per block, the last one possibly short).
inline int blk_row(int b, int h) { return b * kCholBlock < h ? b * kCholBlock : h; }

// Right-hand sides of the triangular solves: per layer an h x nc fp32 matrix
// (row stride nc) at R + layer * stride; layers whose mask entry is 0 are
// left untouched (no mask: all layers). lower: the right-hand side is lower
// triangular (the identity, for L^-1), so a forward solve keeps row block
// [r0, r2) zero from column r2 on and the products skip those columns (the
// columns they would touch are exact zeros either way: same results).
struct Rhs {
  float* R;
  int nc;
  int64_t stride;
  const int* mask;
  bool lower = false;
};

// Rows of blocks [ba, bb) of the right-hand sides <- L^-1 R for the
// lower-triangular factor in w.L.
hipError_t solve_lower(int ba, int bb, const RidgeWs& w, const Rhs& r, int h, int L,
                       hipStream_t s) {
  const int64_t hh = static_cast<int64_t>(h) * h;
  const int64_t lb = static_cast<int64_t>(h) * kCholBlock;
  const int r0 = blk_row(ba, h), r2 = blk_row(bb, h);
  if (bb - ba == 1) {
    float* rk = r.R + static_cast<int64_t>(r0) * r.nc;
    const float* linv = w.Linv + static_cast<int64_t>(r0) * kCholBlock;
    const int nbk = r2 - r0;
    return gemm(nbk, r.lower ? r2 : r.nc, nbk, linv, kCholBlock, 1, lb, false, rk, r.nc, 1,
                r.stride, false, rk, r.nc, r.stride, 1.f, 0.f, L, false, s, r.mask);
  }
  const int bm = (ba + bb) / 2, r1 = blk_row(bm, h);
  hipError_t e = solve_lower(ba, bm, w, r, h, L, s);
  if (e != hipSuccess) return e;
  // R[r1:r2] -= L[r1:r2, r0:r1] R[r0:r1]
  e = gemm(r2 - r1, r.lower ? r1 : r.nc, r1 - r0, w.L + static_cast<int64_t>(r1) * h + r0, h, 1,
           hh, false, r.R + static_cast<int64_t>(r0) * r.nc, r.nc, 1, r.stride, false,
           r.R + static_cast<int64_t>(r1) * r.nc, r.nc, r.stride, -1.f, 1.f, L, false, s, r.mask);
  if (e != hipSuccess) return e;
  return solve_lower(bm, bb, w, r, h, L, s);
}

// Rows of blocks [ba, bb) of the right-hand sides <- L^-T R.
hipError_t solve_upper(int ba, int bb, const RidgeWs& w, const Rhs& r, int h, int L,
                       hipStream_t s) {
  const int64_t hh = static_cast<int64_t>(h) * h;
  const int64_t lb = static_cast<int64_t>(h) * kCholBlock;
  const int r0 = blk_row(ba, h), r2 = blk_row(bb, h);
  if (bb - ba == 1) {
    float* rk = r.R + static_cast<int64_t>(r0) * r.nc;
    const float* linv = w.Linv + static_cast<int64_t>(r0) * kCholBlock;
    const int nbk = r2 - r0;
    return gemm(nbk, r.nc, nbk, linv, 1, kCholBlock, lb, false, rk, r.nc, 1, r.stride, false, rk,
                r.nc, r.stride, 1.f, 0.f, L, false, s, r.mask);
  }
  const int bm = (ba + bb) / 2, r1 = blk_row(bm, h);
  hipError_t e = solve_upper(bm, bb, w, r, h, L, s);
  if (e != hipSuccess) return e;
  // R[r0:r1] -= L[r1:r2, r0:r1]^T R[r1:r2]
  e = gemm(r1 - r0, r.nc, r2 - r1, w.L + static_cast<int64_t>(r1) * h + r0, 1, h, hh, false,
           r.R + static_cast<int64_t>(r1) * r.nc, r.nc, 1, r.stride, false,
           r.R + static_cast<int64_t>(r0) * r.nc, r.nc, r.stride, -1.f, 1.f, L, false, s, r.mask);
  if (e != hipSuccess) return e;
  return solve_upper(ba, bm, w, r, h, L, s);
}

// Columns of blocks [ca, cb) of the rows [x0, x1) of w.L: X <- X L^-T for the
// lower-triangular diagonal part L[blocks ca..cb) (already factored, with the
// diagonal-block inverses in w.Linv).
hipError_t solve_right(int ca, int cb, int x0, int x1, const RidgeWs& w, int h, int L,
                       hipStream_t s) {
  const int64_t hh = static_cast<int64_t>(h) * h;
  const int64_t lb = static_cast<int64_t>(h) * kCholBlock;
  const int c0 = blk_row(ca, h), c2 = blk_row(cb, h);
  float* x = w.L + static_cast<int64_t>(x0) * h;
  if (cb - ca == 1) {
    // X_k <- X_k Linv_kk^T   (in place: one tile column)
    const float* linv = w.Linv + static_cast<int64_t>(c0) * kCholBlock;
    const int nbk = c2 - c0;
    return gemm(x1 - x0, nbk, nbk, x + c0, h, 1, hh, false, linv, 1, kCholBlock, lb, false,
                x + c0, h, hh, 1.f, 0.f, L, false, s);
  }
  const int cm = (ca + cb) / 2, c1 = blk_row(cm, h);
  hipError_t e = solve_right(ca, cm, x0, x1, w, h, L, s);
  if (e != hipSuccess) return e;
  // X[:, c1:c2] -= X[:, c0:c1] L[c1:c2, c0:c1]^T
  e = gemm(x1 - x0, c2 - c1, c1 - c0, x + c0, h, 1, hh, false,
           w.L + static_cast<int64_t>(c1) * h + c0, 1, h, hh, false, x + c1, h, hh, -1.f, 1.f, L,
           false, s);
  if (e != hipSuccess) return e;
  return solve_right(cm, cb, x0, x1, w, h, L, s);
}

// Cholesky factor of the diagonal blocks [ba, bb) of w.L (their trailing
// updates from earlier columns already applied).
hipError_t cholesky(int ba, int bb, const RidgeWs& w, int h, int L, int* info, hipStream_t s) {
  const int64_t hh = static_cast<int64_t>(h) * h;
  const int r0 = blk_row(ba, h), r2 = blk_row(bb, h);
  if (bb - ba == 1) return ispa::launch_potrf_block(w.L, w.Linv, h, r0, r2 - r0, L, info, ba == 0, s);
  const int bm = (ba + bb) / 2, r1 = blk_row(bm, h);
  hipError_t e = cholesky(ba, bm, w, h, L, info, s);
  if (e != hipSuccess) return e;
  // L21 = A21 L11^-T
  e = solve_right(ba, bm, r1, r2, w, h, L, s);
  if (e != hipSuccess) return e;
  // A22 -= L21 L21^T   (lower 128-tiles only)
  float* l21 = w.L + static_cast<int64_t>(r1) * h + r0;
  e = gemm(r2 - r1, r2 - r1, r1 - r0, l21, h, 1, hh, false, l21, 1, h, hh, false,
           w.L + static_cast<int64_t>(r1) * h + r1, h, hh, -1.f, 1.f, L, true, s);
  if (e != hipSuccess) return e;
  return cholesky(bm, bb, w, h, L, info, s);
}

}  // namespace

extern "C" {

const char* ispa_status_string(int status) {
  switch (status) {
    case ISPA_OK: return "ok";
    case ISPA_ERR_NULL: return "required pointer is NULL";
    case ISPA_ERR_SHAPE: return "size out of range or inconsistent";
    case ISPA_ERR_UNSUPPORTED: return "unsupported configuration";
    case ISPA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case ISPA_ERR_WORKSPACE: return "workspace missing or too small";
    case ISPA_ERR_HIP: return "HIP runtime error (launch, copy or memory mapping)";
    case ISPA_ERR_SCRATCH: return "input exceeds the fixed scratch of an allocation-free entry point";
    default: return "unknown status";
  }
}

int ispa_version(void) { return 100; }

}  // extern "C"

namespace {

// Validation and parameters shared by the bf16 and E4M3 attention entry
// points. Returns ISPA_OK with *run = false when there is nothing to do.
int attn_setup(const void* q, int64_t n_q, const void* k_sink, const void* v_sink,
               int64_t n_sink, const void* k_cur, const void* v_cur, int64_t n_cur,
               const void* k_hist, const void* v_hist, int64_t n_hist, int n_heads,
               int head_dim, float sm_scale, void* o_local, float* lse_local, void* o_hist,
               float* lse_hist, void* o_full, float* lse_full, void* d_out,
               ispa::AttnParams* out, bool* run, void* xt = nullptr, void* dt = nullptr,
               int64_t ldt = 0, const void* k_hist2 = nullptr, const void* v_hist2 = nullptr,
               int64_t n_hist2 = 0) {
  *run = false;
  if (n_q < 0 || n_sink < 0 || n_cur < 0 || n_hist < 0 || n_hist2 < 0 || n_heads < 1)
    return ISPA_ERR_SHAPE;
  if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return ISPA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return ISPA_ERR_UNSUPPORTED;
  if (!q && n_q > 0) return ISPA_ERR_NULL;
  if ((n_sink > 0 && (!k_sink || !v_sink)) || (n_cur > 0 && (!k_cur || !v_cur)) ||
      (n_hist > 0 && (!k_hist || !v_hist)) || (n_hist2 > 0 && (!k_hist2 || !v_hist2)))
    return ISPA_ERR_NULL;
  if (!o_local && !lse_local && !o_hist && !lse_hist && !o_full && !lse_full && !d_out && !xt &&
      !dt)
    return ISPA_ERR_NULL;
  if (n_sink + n_cur < 1) return ISPA_ERR_SHAPE;
  const void* ptrs[] = {q,         k_sink,   v_sink, k_cur,  v_cur,    k_hist,
                        v_hist,    k_hist2,  v_hist2, o_local, lse_local, o_hist,
                        lse_hist,  o_full,   lse_full, d_out,  xt,       dt};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return ISPA_ERR_ALIGN;
  const int64_t qtiles = (n_q + ispa::attn_q_tile_min() - 1) / ispa::attn_q_tile_min();
  if (qtiles * n_heads > INT32_MAX) return ISPA_ERR_SHAPE;
  if (n_q == 0) return ISPA_OK;

  ispa::AttnParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k[0] = static_cast<const uint16_t*>(k_sink);
  p.v[0] = static_cast<const uint16_t*>(v_sink);
  p.n[0] = n_sink;
  p.k[1] = static_cast<const uint16_t*>(k_cur);
  p.v[1] = static_cast<const uint16_t*>(v_cur);
  p.n[1] = n_cur;
  p.k[2] = static_cast<const uint16_t*>(k_hist);
  p.v[2] = static_cast<const uint16_t*>(v_hist);
  p.n[2] = n_hist;
  p.k[3] = static_cast<const uint16_t*>(k_hist2);
  p.v[3] = static_cast<const uint16_t*>(v_hist2);
  p.n[3] = n_hist2;
  p.n_q = n_q;
  p.n_heads = n_heads;
  p.scale_log2 = static_cast<float>(static_cast<double>(sm_scale) * 1.4426950408889634);
  p.o_local = static_cast<uint16_t*>(o_local);
  p.lse_local = lse_local;
  p.o_hist = static_cast<uint16_t*>(o_hist);
  p.lse_hist = lse_hist;
  p.o_full = static_cast<uint16_t*>(o_full);
  p.lse_full = lse_full;
  p.d_out = static_cast<uint16_t*>(d_out);
  p.xt = static_cast<uint16_t*>(xt);
  p.dt = static_cast<uint16_t*>(dt);
  p.ldt = ldt;
  const bool only_full = !o_local && !lse_local && !o_hist && !lse_hist && !d_out && !xt && !dt;
  p.mode = only_full ? 1 : 0;
  p.need_hist = (o_hist || lse_hist || o_full || lse_full || d_out || dt) ? 1 : 0;
  *out = p;
  *run = true;
  return ISPA_OK;
}

}  // namespace

namespace ispa {

int attn_decomp_two_piece_history(const void* q, int64_t n_q, const void* k_sink,
                                  const void* v_sink, int64_t n_sink, const void* k_cur,
                                  const void* v_cur, int64_t n_cur, const void* k_hist,
                                  const void* v_hist, int64_t n_hist, const void* k_hist2,
                                  const void* v_hist2, int64_t n_hist2, int n_heads, int head_dim,
                                  float sm_scale, void* o_local, float* lse_local, void* o_hist,
                                  float* lse_hist, void* o_full, float* lse_full, void* d_out,
                                  void* stream) {
  AttnParams p{};
  bool run = false;
  const int st = attn_setup(q, n_q, k_sink, v_sink, n_sink, k_cur, v_cur, n_cur, k_hist, v_hist,
                            n_hist, n_heads, head_dim, sm_scale, o_local, lse_local, o_hist,
                            lse_hist, o_full, lse_full, d_out, &p, &run, nullptr, nullptr, 0,
                            k_hist2, v_hist2, n_hist2);
  if (st != ISPA_OK || !run) return st;
  return hip_status(launch_attn_decomp(p, head_dim, as_stream(stream)));
}

}  // namespace ispa

namespace {

// Workspace of the E4M3 attention: query codes, scales and shifts, then per
// segment the key codes and tile scales.
struct AttnFp8Ws {
  uint8_t* q8;
  float* qsc;
  float* qmu;
  uint8_t* k8[3];
  float* ksc[3];
  size_t bytes;
};

AttnFp8Ws attn_fp8_layout(void* base, int64_t n_q, const int64_t n[3], int n_heads) {
  AttnFp8Ws w{};
  const size_t row = static_cast<size_t>(n_heads) * 128;
  char* p = static_cast<char*>(base);
  size_t off = 0;
  w.q8 = reinterpret_cast<uint8_t*>(p + off);  off = align_up(off + n_q * row);
  w.qsc = reinterpret_cast<float*>(p + off);   off = align_up(off + n_q * n_heads * 4);
  w.qmu = reinterpret_cast<float*>(p + off);   off = align_up(off + n_q * n_heads * 4);
  for (int g = 0; g < 3; ++g) {
    w.k8[g] = reinterpret_cast<uint8_t*>(p + off);
    off = align_up(off + n[g] * row);
    w.ksc[g] = reinterpret_cast<float*>(p + off);
    off = align_up(off + ispa::key_tiles(n[g]) * n_heads * 4);
  }
  w.bytes = off;
  return w;
}

}  // namespace

extern "C" {

int ispa_attn_decomp(const void* q, int64_t n_q, const void* k_sink, const void* v_sink,
                     int64_t n_sink, const void* k_cur, const void* v_cur, int64_t n_cur,
                     const void* k_hist, const void* v_hist, int64_t n_hist, int n_heads,
                     int head_dim, float sm_scale, void* o_local, float* lse_local, void* o_hist,
                     float* lse_hist, void* o_full, float* lse_full, void* d_out, void* stream) {
  ispa::AttnParams p{};
  bool run = false;
  const int st = attn_setup(q, n_q, k_sink, v_sink, n_sink, k_cur, v_cur, n_cur, k_hist, v_hist,
                            n_hist, n_heads, head_dim, sm_scale, o_local, lse_local, o_hist,
                            lse_hist, o_full, lse_full, d_out, &p, &run);
  if (st != ISPA_OK || !run) return st;
  return hip_status(ispa::launch_attn_decomp(p, head_dim, as_stream(stream)));
}

int ispa_attn_decomp_t(const void* q, int64_t n_q, const void* k_sink, const void* v_sink,
                       int64_t n_sink, const void* k_cur, const void* v_cur, int64_t n_cur,
                       const void* k_hist, const void* v_hist, int64_t n_hist, int n_heads,
                       int head_dim, float sm_scale, void* o_full, float* lse_full, void* xt,
                       void* dt, int64_t ld, void* stream) {
  if (!xt || !dt || !o_full) return ISPA_ERR_NULL;
  if (ld < n_q || ld < 1) return ISPA_ERR_SHAPE;
  if (ld % 8 != 0) return ISPA_ERR_ALIGN;
  // the feature-major outputs are addressed with 32-bit byte offsets
  if (static_cast<int64_t>(n_heads) * head_dim * ld * 2 > INT32_MAX) return ISPA_ERR_UNSUPPORTED;
  ispa::AttnParams p{};
  bool run = false;
  const int st = attn_setup(q, n_q, k_sink, v_sink, n_sink, k_cur, v_cur, n_cur, k_hist, v_hist,
                            n_hist, n_heads, head_dim, sm_scale, nullptr, nullptr, nullptr,
                            nullptr, o_full, lse_full, nullptr, &p, &run, xt, dt, ld);
  if (st != ISPA_OK || !run) return st;
  return hip_status(ispa::launch_attn_decomp(p, head_dim, as_stream(stream)));
}

int ispa_attn_decomp_grouped(const ispa_attn_job* jobs, int n_jobs, int n_heads, int head_dim,
                             float sm_scale, void* stream) {
  if (!jobs) return ISPA_ERR_NULL;
  if (n_jobs < 1 || n_jobs > ISPA_MAX_GROUP) return ISPA_ERR_SHAPE;
  ispa::AttnGroup grp{};
  for (int g = 0; g < n_jobs; ++g) {
    const ispa_attn_job& j = jobs[g];
    if (j.n_q == 0) continue;  // nothing to compute (its outputs may be empty, i.e. NULL)
    ispa::AttnParams p{};
    bool run = false;
    const int st = attn_setup(j.q, j.n_q, j.k_sink, j.v_sink, j.n_sink, j.k_cur, j.v_cur,
                              j.n_cur, j.k_hist, j.v_hist, j.n_hist, n_heads, head_dim, sm_scale,
                              j.o_local, j.lse_local, j.o_hist, j.lse_hist, j.o_full, j.lse_full,
                              j.d_out, &p, &run);
    if (st != ISPA_OK) return st;
    if (run) grp.p[grp.n++] = p;
  }
  if (grp.n == 0) return ISPA_OK;
  // A call whose own grid covers at least half the compute units runs as a
  // launch of its own: grouping it saves little idle hardware and adds tail
  // imbalance between calls of different lengths. The smaller calls share
  // one launch.
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return ISPA_ERR_HIP;
  const hipStream_t s = as_stream(stream);
  ispa::AttnGroup small{};
  for (int g = 0; g < grp.n; ++g) {
    const int64_t tiles = (grp.p[g].n_q + ispa::attn_q_tile_min() - 1) / ispa::attn_q_tile_min();
    if (tiles * n_heads >= cus / 2)
      ISPA_TRY(ispa::launch_attn_decomp(grp.p[g], head_dim, s));
    else
      small.p[small.n++] = grp.p[g];
  }
  if (small.n == 1) return hip_status(ispa::launch_attn_decomp(small.p[0], head_dim, s));
  if (small.n == 0) return ISPA_OK;
  return hip_status(ispa::launch_attn_grouped(small, head_dim, s));
}

size_t ispa_attn_fp8_workspace_bytes(int64_t n_q, int64_t n_sink, int64_t n_cur, int64_t n_hist,
                                     int n_heads, int head_dim) {
  if (n_q < 0 || n_sink < 0 || n_cur < 0 || n_hist < 0 || n_heads < 1 || head_dim != 128)
    return 0;
  const int64_t n[3] = {n_sink, n_cur, n_hist};
  return attn_fp8_layout(nullptr, n_q, n, n_heads).bytes;
}

int ispa_attn_decomp_fp8(const void* q, int64_t n_q, const void* k_sink, const void* v_sink,
                         int64_t n_sink, const void* k_cur, const void* v_cur, int64_t n_cur,
                         const void* k_hist, const void* v_hist, int64_t n_hist, int n_heads,
                         int head_dim, float sm_scale, const void* k_mean, void* o_local,
                         float* lse_local, void* o_hist, float* lse_hist, void* o_full,
                         float* lse_full, void* d_out, void* workspace, size_t ws_bytes,
                         void* stream) {
  ispa::AttnParams p{};
  bool run = false;
  const int st = attn_setup(q, n_q, k_sink, v_sink, n_sink, k_cur, v_cur, n_cur, k_hist, v_hist,
                            n_hist, n_heads, head_dim, sm_scale, o_local, lse_local, o_hist,
                            lse_hist, o_full, lse_full, d_out, &p, &run);
  if (st != ISPA_OK) return st;
  if (head_dim != 128) return ISPA_ERR_UNSUPPORTED;
  if (k_mean && !aligned16(k_mean)) return ISPA_ERR_ALIGN;
  // one quantization workgroup per (64-key tile, head) and one per 4 query rows
  for (const int64_t nk : {n_sink, n_cur, n_hist})
    if (ispa::key_tiles(nk) * n_heads > INT32_MAX) return ISPA_ERR_SHAPE;
  if ((n_q * n_heads + 3) / 4 > INT32_MAX) return ISPA_ERR_SHAPE;
  if (!run) return ISPA_OK;
  if (!workspace ||
      ws_bytes < ispa_attn_fp8_workspace_bytes(n_q, n_sink, n_cur, n_hist, n_heads, head_dim))
    return ISPA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ISPA_ERR_ALIGN;
  const int64_t n[3] = {n_sink, n_cur, n_hist};
  const AttnFp8Ws w = attn_fp8_layout(workspace, n_q, n, n_heads);
  const hipStream_t s = as_stream(stream);
  const uint16_t* mu = static_cast<const uint16_t*>(k_mean);
  ISPA_TRY(ispa::launch_quantize_queries_fp8(p.q, n_q, n_heads, mu, sm_scale, w.q8, w.qsc,
                                             mu ? w.qmu : nullptr, s));
  for (int g = 0; g < 3; ++g)
    ISPA_TRY(ispa::launch_quantize_key_tiles_fp8(p.k[g], n[g], n_heads, mu, w.k8[g], w.ksc[g],
                                                 s));
  p.q8 = w.q8;
  p.qsc = w.qsc;
  p.qmu = mu ? w.qmu : nullptr;
  for (int g = 0; g < 3; ++g) {
    p.k8[g] = w.k8[g];
    p.ksc[g] = w.ksc[g];
  }
  return hip_status(ispa::launch_attn_decomp(p, head_dim, s));
}

size_t ispa_key_mean_workspace_bytes(int n_heads, int head_dim) {
  if (n_heads < 1 || head_dim != 128) return 0;
  return static_cast<size_t>(ispa::key_mean_splits()) * n_heads * head_dim * sizeof(float);
}

int ispa_key_mean(const void* k_sink, int64_t n_sink, const void* k_cur, int64_t n_cur,
                  const void* k_hist, int64_t n_hist, int n_heads, int head_dim, void* mu,
                  void* workspace, size_t ws_bytes, void* stream) {
  if (!mu) return ISPA_ERR_NULL;
  if (n_sink < 0 || n_cur < 0 || n_hist < 0 || n_heads < 1) return ISPA_ERR_SHAPE;
  if ((n_sink > 0 && !k_sink) || (n_cur > 0 && !k_cur) || (n_hist > 0 && !k_hist))
    return ISPA_ERR_NULL;
  if (n_sink + n_cur + n_hist < 1) return ISPA_ERR_SHAPE;
  if (head_dim != 128) return ISPA_ERR_UNSUPPORTED;
  if (!workspace || ws_bytes < ispa_key_mean_workspace_bytes(n_heads, head_dim))
    return ISPA_ERR_WORKSPACE;
  const void* ptrs[] = {k_sink, k_cur, k_hist, mu, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return ISPA_ERR_ALIGN;
  ispa::KeySegs segs{};
  segs.k[0] = static_cast<const uint16_t*>(k_sink);
  segs.k[1] = static_cast<const uint16_t*>(k_cur);
  segs.k[2] = static_cast<const uint16_t*>(k_hist);
  segs.n[0] = n_sink;
  segs.n[1] = n_cur;
  segs.n[2] = n_hist;
  return hip_status(ispa::launch_key_mean(segs, n_heads, static_cast<float*>(workspace),
                                          static_cast<uint16_t*>(mu), as_stream(stream)));
}

int ispa_gram_accumulate(const void* x, const void* d, int64_t n_tok, int h, int n_batch,
                         float* G, float* C, float* E, int zero_first, void* stream) {
  if (!x || !d || !G || !C) return ISPA_ERR_NULL;
  if (h < 1 || n_tok < 0 || n_batch < 1) return ISPA_ERR_SHAPE;
  if (h % 8 != 0) return ISPA_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(d) || !aligned16(G) || !aligned16(C) || (E && !aligned16(E)))
    return ISPA_ERR_ALIGN;
  ispa::GramParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.d = static_cast<const uint16_t*>(d);
  p.n_tok = n_tok;
  p.h = h;
  p.batch = n_batch;
  p.G = G;
  p.C = C;
  p.E = E;
  p.zero_first = zero_first ? 1 : 0;
  if (n_tok == 0 && !zero_first) return ISPA_OK;
  return hip_status(ispa::launch_gram(p, as_stream(stream)));
}

int ispa_gram_accumulate_t(const void* xt, const void* dt, int64_t n_tok, int64_t ld, int h,
                           int n_batch, float* G, float* C, float* E, int zero_first,
                           void* stream) {
  if (!xt || !dt || !G || !C) return ISPA_ERR_NULL;
  if (h < 1 || n_tok < 0 || n_batch < 1 || ld < n_tok || ld < 1) return ISPA_ERR_SHAPE;
  if (h % 8 != 0) return ISPA_ERR_UNSUPPORTED;
  if (ld % 8 != 0 || !aligned16(xt) || !aligned16(dt) || !aligned16(G) || !aligned16(C) ||
      (E && !aligned16(E)))
    return ISPA_ERR_ALIGN;
  // buffer offsets of the loads are 32-bit: one layer's X^T must stay below 2 GiB
  if (static_cast<int64_t>(h) * ld * 2 > INT32_MAX || n_tok > INT32_MAX)
    return ISPA_ERR_UNSUPPORTED;
  if (n_tok == 0 && !zero_first) return ISPA_OK;
  return hip_status(ispa::launch_gram_t(static_cast<const uint16_t*>(xt),
                                        static_cast<const uint16_t*>(dt), n_tok, ld, h, n_batch, G,
                                        C, E, zero_first, as_stream(stream)));
}

size_t ispa_ridge_workspace_bytes(int n_layers, int h) {
  if (n_layers < 1 || h < 1) return 0;
  return ridge_layout(nullptr, n_layers, h).bytes;
}

int ispa_ridge_solve(int n_layers, int h, const float* G, const float* C, const void* Wo,
                     float lambda, float* dW, int* info, void* workspace, size_t ws_bytes,
                     void* stream) {
  if (!G || !C || !Wo || !dW || !info) return ISPA_ERR_NULL;
  if (n_layers < 1 || h < 1 || !(lambda >= 0.f) || !isfinite(lambda)) return ISPA_ERR_SHAPE;
  if (h % 8 != 0) return ISPA_ERR_UNSUPPORTED;
  if (!workspace || ws_bytes < ispa_ridge_workspace_bytes(n_layers, h)) return ISPA_ERR_WORKSPACE;
  if (!aligned16(G) || !aligned16(C) || !aligned16(Wo) || !aligned16(dW) || !aligned16(info) ||
      !aligned16(workspace))
    return ISPA_ERR_ALIGN;
  const hipStream_t s = as_stream(stream);
  const RidgeWs w = ridge_layout(workspace, n_layers, h);
  const int64_t hh = static_cast<int64_t>(h) * h;
  const int L = n_layers;
  const int nblk = (h + kCholBlock - 1) / kCholBlock;

  // Cholesky of M = G + lambda I by recursive halving over the 128-column
  // blocks (leaves factor and invert one diagonal block; panels are solved
  // against the leaves' inverses; trailing updates are single large
  // lower-tile products).
  ISPA_TRY(ispa::launch_copy_add_diag(G, w.L, h, L, lambda, s));
  ISPA_TRY(cholesky(0, nblk, w, h, L, info, s));

  // Y0 = (G + lambda I)^-1 C by forward substitution L Z = C and back
  // substitution L^T Y0 = Z, both by recursive halving over the 128-row
  // blocks: solve one half, update the other half with one large GEMM (K up
  // to h/2), solve it. The leaves apply the diagonal-block inverses in place.
  // Compared with block-row sweeps this touches each row of the right-hand
  // side O(log(h/128)) times instead of O(h/128) times, and the update GEMMs
  // are large.
  ISPA_TRY(hipMemcpyAsync(w.R, C, static_cast<size_t>(L) * hh * sizeof(float),
                          hipMemcpyDeviceToDevice, s));
  const Rhs ry{w.R, h, hh, nullptr};
  ISPA_TRY(solve_lower(0, nblk, w, ry, h, L, s));
  ISPA_TRY(solve_upper(0, nblk, w, ry, h, L, s));

  // Iterative refinement, one step, for the layers that need it. The fp32
  // factor solves to about cond * 2^-24 (1e-3 relative at cond 2e4,
  // rank-deficient statistics: eigenvalues lambda outside the span of the
  // warmup tokens). The system is solved for (G + lambda I)^-1 C rather than
  // for dW directly, so that its right-hand side C is an exact input: C W
  // formed in fp32 would carry a rounding of 2^-24 |C| |W| that no
  // refinement of the solve can remove, and the multiplication by W after the
  // solve is well conditioned.
  //
  // Which layers: the error of dW0 = Y0 W along 8 random directions,
  // E W z = (G + lambda I)^-1 (C W z - (G + lambda I) Y0 W z), with the
  // residual accumulated in fp64 and solved with the same factor; for
  // Gaussian-like z its squared norm estimates ||E W||_F^2. A layer is refined
  // unless that estimate is below kRefineTol relative to ||Y0 W z||. Cost:
  // three fp64 matrix-vector passes and one 8-column solve per layer.
  ISPA_TRY(ispa::launch_probe_wz(static_cast<const uint16_t*>(Wo), w.pq, h, L, s));
  ISPA_TRY(ispa::launch_mv8_f64(C, w.pq, w.pa, h, L, s));
  ISPA_TRY(ispa::launch_mv8_f64(w.R, w.pq, w.pb, h, L, s));
  ISPA_TRY(ispa::launch_mv8_f64(G, w.pb, w.pt, h, L, s));
  ISPA_TRY(ispa::launch_probe_resid(w.pa, w.pt, w.pb, static_cast<double>(lambda), w.pe, h, L, s));
  const Rhs rp8{w.pe, 8, static_cast<int64_t>(h) * 8, nullptr};
  ISPA_TRY(solve_lower(0, nblk, w, rp8, h, L, s));
  ISPA_TRY(solve_upper(0, nblk, w, rp8, h, L, s));
  ISPA_TRY(ispa::launch_probe_flag(w.pe, w.pb, kRefineTol, w.refine, h, L, s));

  // The step: the residual S = C - (G + lambda I) Y0 accumulated in fp64,
  // the correction (G + lambda I)^-1 S from the same factor, Y = Y0 +
  // correction: about (cond * 2^-24)^2. Layers not flagged skip all three.
  {
    ispa::RidgeResidParams rp{};
    rp.h = h;
    rp.batch = L;
    rp.G = G;
    rp.C = C;
    rp.Y = w.R;
    rp.S = w.S;
    rp.lam = static_cast<double>(lambda);
    rp.layer_mask = w.refine;
    ISPA_TRY(ispa::launch_ridge_resid_f64(rp, s));
  }
  const Rhs rs{w.S, h, hh, w.refine};
  ISPA_TRY(solve_lower(0, nblk, w, rs, h, L, s));
  ISPA_TRY(solve_upper(0, nblk, w, rs, h, L, s));
  ISPA_TRY(ispa::launch_add_inplace(w.R, w.S, hh, L, w.refine, s));

  // dW (math layout [in, out]) = Y W, W(k, o) = Wo[o][k]: dW[i][o] =
  // sum_k Y[i][k] Wo[o][k] on the bf16 matrix cores with Y split into two
  // bf16 planes (hi + lo holds Y to ~2^-17 relative per element; the errors
  // are independent and stay at that level in the product), staged in Bt;
  // then the transpose into the caller's nn.Linear layout.
  {
    uint16_t* yhi = reinterpret_cast<uint16_t*>(w.Bt);
    uint16_t* ylo = yhi + static_cast<int64_t>(L) * hh;
    ISPA_TRY(ispa::launch_split_nt_gemm_f32(w.R, yhi, ylo, static_cast<const uint16_t*>(Wo), w.S,
                                            h, L, s));
  }
  ISPA_TRY(ispa::launch_transpose(w.S, dW, h, L, s));
  // (C W)^T in nn.Linear layout for the layer score, the same way.
  {
    uint16_t* chi = reinterpret_cast<uint16_t*>(w.Bt);
    uint16_t* clo = chi + static_cast<int64_t>(L) * hh;
    ISPA_TRY(ispa::launch_split_nt_gemm_f32(C, chi, clo, static_cast<const uint16_t*>(Wo), w.R, h,
                                            L, s));
  }
  ISPA_TRY(ispa::launch_transpose(w.R, w.Bt, h, L, s));
  return ISPA_OK;
}

int ispa_layer_score(int n_layers, int h, const float* G, const float* C, const float* E,
                     const void* Wo, const float* dW, float lambda, const int* info, int K,
                     void* workspace, size_t ws_bytes, double* eps_abs, double* eps_rel,
                     int* selected, void* stream) {
  if (!G || !C || !E || !Wo || !dW || !eps_abs || !eps_rel || !selected) return ISPA_ERR_NULL;
  if (n_layers < 1 || h < 1 || K < 0 || !(lambda >= 0.f) || !isfinite(lambda))
    return ISPA_ERR_SHAPE;
  if (h % 8 != 0) return ISPA_ERR_UNSUPPORTED;
  if (!workspace || ws_bytes < ispa_ridge_workspace_bytes(n_layers, h)) return ISPA_ERR_WORKSPACE;
  if (!aligned16(G) || !aligned16(C) || !aligned16(E) || !aligned16(Wo) || !aligned16(dW) ||
      !aligned16(workspace) || !aligned16(eps_abs) || !aligned16(eps_rel) || !aligned16(selected) ||
      (info && !aligned16(info)))
    return ISPA_ERR_ALIGN;
  const hipStream_t s = as_stream(stream);
  const RidgeWs w = ridge_layout(workspace, n_layers, h);
  const int64_t hh = static_cast<int64_t>(h) * h;
  // P = W W^T (math W = Wo^T): P(i, j) = sum_o Wo[o][i] Wo[o][j], the Gram of
  // the bf16 rows of Wo, formed on the bf16 matrix cores (products exact in
  // fp32, fp32 accumulation); both triangles are written.
  {
    ispa::GramParams gp{};
    gp.x = static_cast<const uint16_t*>(Wo);
    gp.d = nullptr;
    gp.n_tok = h;
    gp.h = h;
    gp.batch = n_layers;
    gp.G = w.L;
    gp.zero_first = 1;
    ISPA_TRY(ispa::launch_gram(gp, s));
  }
  ispa::ScoreParams p{};
  p.n_layers = n_layers;
  p.h = h;
  p.G = G;
  p.C = C;
  p.E = E;
  p.Wo = static_cast<const uint16_t*>(Wo);
  p.dW = dW;
  p.lam = lambda;
  p.info = info;
  p.K = K;
  p.partial = w.part;
  p.eps_abs = eps_abs;
  p.eps_rel = eps_rel;
  p.selected = selected;
  return hip_status(ispa::launch_score(p, w.L, w.Bt, s));
}

int ispa_apply_dW(int n_layers, int h, const int* selected, const float* dW, void* Wo,
                  void* stream) {
  if (!selected || !dW || !Wo) return ISPA_ERR_NULL;
  if (n_layers < 1 || h < 1) return ISPA_ERR_SHAPE;
  if (h % 8 != 0) return ISPA_ERR_UNSUPPORTED;
  if (!aligned16(selected) || !aligned16(dW) || !aligned16(Wo)) return ISPA_ERR_ALIGN;
  return hip_status(ispa::launch_apply_dw(n_layers, h, selected, dW,
                                          static_cast<uint16_t*>(Wo), as_stream(stream)));
}

size_t ispa_drift_workspace_bytes(int n_layers, int h, int64_t n_sample) {
  if (n_layers < 1 || h < 1 || n_sample < 1) return 0;
  const size_t ridge = ridge_layout(nullptr, n_layers, h).bytes;
  const size_t y = align_up(static_cast<size_t>(n_layers) * h * n_sample * sizeof(float)) +
                   align_up(static_cast<size_t>(n_layers) * ispa::drift_partial_count(h) *
                            sizeof(double));
  return ridge > y ? ridge : y;
}

int ispa_drift_prepare(int n_layers, int h, const float* G, float lambda, int64_t n_warm,
                       float* linv, double* ref, int* info, void* workspace, size_t ws_bytes,
                       void* stream) {
  if (!G || !linv || !ref || !info) return ISPA_ERR_NULL;
  if (n_layers < 1 || h < 1 || n_warm < 1 || !(lambda >= 0.f) || !isfinite(lambda))
    return ISPA_ERR_SHAPE;
  if (h % 8 != 0) return ISPA_ERR_UNSUPPORTED;
  if (!workspace || ws_bytes < ridge_layout(nullptr, n_layers, h).bytes) return ISPA_ERR_WORKSPACE;
  if (!aligned16(G) || !aligned16(linv) || !aligned16(ref) || !aligned16(info) ||
      !aligned16(workspace))
    return ISPA_ERR_ALIGN;
  const hipStream_t s = as_stream(stream);
  const RidgeWs w = ridge_layout(workspace, n_layers, h);
  const int nblk = (h + kCholBlock - 1) / kCholBlock;
  const int64_t hh = static_cast<int64_t>(h) * h;
  ISPA_TRY(ispa::launch_copy_add_diag(G, w.L, h, n_layers, lambda, s));
  ISPA_TRY(cholesky(0, nblk, w, h, n_layers, info, s));
  ISPA_TRY(ispa::launch_identity(linv, h, n_layers, s));
  ISPA_TRY(solve_lower(0, nblk, w, Rhs{linv, h, hh, nullptr, true}, h, n_layers, s));
  // ||L^{-1}||_F^2 = tr((G + lambda I)^{-1}) -> (h - lambda tr) / n_warm
  ISPA_TRY(ispa::launch_drift_sum(linv, h, h, h, hh, n_layers, w.part, h, lambda,
                                  static_cast<double>(n_warm), nullptr, ref, s));
  return ISPA_OK;
}

int ispa_drift_prepare_factored(int n_layers, int h, float lambda, int64_t n_warm, float* linv,
                                double* ref, void* workspace, size_t ws_bytes, void* stream) {
  if (!linv || !ref || !workspace) return ISPA_ERR_NULL;
  if (n_layers < 1 || h < 1 || n_warm < 1 || !(lambda >= 0.f) || !isfinite(lambda))
    return ISPA_ERR_SHAPE;
  if (h % 8 != 0) return ISPA_ERR_UNSUPPORTED;
  if (ws_bytes < ridge_layout(nullptr, n_layers, h).bytes) return ISPA_ERR_WORKSPACE;
  if (!aligned16(linv) || !aligned16(ref) || !aligned16(workspace)) return ISPA_ERR_ALIGN;
  // the factor and its diagonal-block inverses are where ispa_ridge_solve
  // left them; only the forward solve L Z = I and the trace remain
  const RidgeWs w = ridge_layout(workspace, n_layers, h);
  const hipStream_t s = as_stream(stream);
  const int nblk = (h + kCholBlock - 1) / kCholBlock;
  const int64_t hh = static_cast<int64_t>(h) * h;
  ISPA_TRY(ispa::launch_identity(linv, h, n_layers, s));
  ISPA_TRY(solve_lower(0, nblk, w, Rhs{linv, h, hh, nullptr, true}, h, n_layers, s));
  ISPA_TRY(ispa::launch_drift_sum(linv, h, h, h, hh, n_layers, w.part, h, lambda,
                                  static_cast<double>(n_warm), nullptr, ref, s));
  return ISPA_OK;
}

int ispa_drift_score(int n_layers, int h, const float* linv, const double* ref, const void* x,
                     int64_t n_tok, int64_t stride, double* score, void* workspace,
                     size_t ws_bytes, void* stream) {
  if (!linv || !ref || !x || !score) return ISPA_ERR_NULL;
  if (n_layers < 1 || h < 1 || n_tok < 1 || stride < 1) return ISPA_ERR_SHAPE;
  if (h % 8 != 0) return ISPA_ERR_UNSUPPORTED;
  const int64_t n_s = (n_tok + stride - 1) / stride;
  if (n_s > INT32_MAX) return ISPA_ERR_SHAPE;
  if (!workspace || ws_bytes < ispa_drift_workspace_bytes(n_layers, h, n_s))
    return ISPA_ERR_WORKSPACE;
  // ref and score are read and written per element: 8-byte alignment, so a
  // layer's entry of a per-layer vector can be passed on its own
  const auto aligned8 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; };
  if (!aligned16(linv) || !aligned8(ref) || !aligned16(x) || !aligned8(score) ||
      !aligned16(workspace))
    return ISPA_ERR_ALIGN;
  const hipStream_t s = as_stream(stream);
  float* Y = static_cast<float*>(workspace);
  double* part = reinterpret_cast<double*>(
      static_cast<char*>(workspace) +
      align_up(static_cast<size_t>(n_layers) * h * n_s * sizeof(float)));
  const int64_t hh = static_cast<int64_t>(h) * h;
  // Y = L^{-1} X_s^T: column j is L^{-1} x^T for sampled token j * stride,
  // so its squared norm is that token's leverage x (G + lambda I)^{-1} x^T
  ISPA_TRY(gemm(h, static_cast<int>(n_s), h, linv, h, 1, hh, false, x, 1, stride * h,
                n_tok * h, true, Y, n_s, h * n_s, 1.f, 0.f, n_layers, false, s));
  ISPA_TRY(ispa::launch_drift_sum(Y, h, static_cast<int>(n_s), n_s, h * n_s, n_layers, part,
                                  h, 0.0, static_cast<double>(n_s), ref, score, s));
  return ISPA_OK;
}

int ispa_quantize_fp8(const void* a, int64_t rows, int k, void* q, float* scale,
                      void* stream) {
  if (!a || !q || !scale) return ISPA_ERR_NULL;
  if (rows < 0 || k < 1 || rows > INT32_MAX) return ISPA_ERR_SHAPE;
  if (k % 8 != 0) return ISPA_ERR_UNSUPPORTED;
  if (!aligned16(a) || !aligned16(q) || !aligned16(scale)) return ISPA_ERR_ALIGN;
  return hip_status(ispa::launch_quantize_rows_fp8(static_cast<const uint16_t*>(a), rows, k,
                                                   static_cast<uint8_t*>(q), scale,
                                                   as_stream(stream)));
}

size_t ispa_project_w8a8_workspace_bytes(int64_t n, int h_in) {
  if (n < 0 || h_in < 1) return 0;
  return align_up(static_cast<size_t>(n) * h_in) + align_up(static_cast<size_t>(n) * 4) + 256;
}

int ispa_project_w8a8(const void* x, const void* wq, const float* w_scale, void* y, int64_t n,
                      int h_in, int h_out, void* workspace, size_t ws_bytes, void* stream) {
  if (!x || !wq || !w_scale || !y) return ISPA_ERR_NULL;
  if (n < 0 || h_in < 1 || h_out < 1 || n > INT32_MAX) return ISPA_ERR_SHAPE;
  if (h_in % 64 != 0 || h_out % 8 != 0) return ISPA_ERR_UNSUPPORTED;
  if (n == 0) return ISPA_OK;
  if (!workspace || ws_bytes < ispa_project_w8a8_workspace_bytes(n, h_in))
    return ISPA_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(wq) || !aligned16(w_scale) || !aligned16(y) ||
      !aligned16(workspace))
    return ISPA_ERR_ALIGN;
  const hipStream_t s = as_stream(stream);
  uint8_t* xq = static_cast<uint8_t*>(workspace);
  float* sx = reinterpret_cast<float*>(xq + align_up(static_cast<size_t>(n) * h_in));
  ISPA_TRY(ispa::launch_quantize_rows_fp8(static_cast<const uint16_t*>(x), n, h_in, xq, sx, s));
  return hip_status(ispa::launch_nt_gemm256_fp8(xq, sx, static_cast<const uint8_t*>(wq),
                                                w_scale, static_cast<uint16_t*>(y), n, h_in,
                                                h_out, s));
}

int ispa_project_grouped(const ispa_project_job* jobs, int n_jobs, int h_in, int h_out,
                         void* stream) {
  if (!jobs) return ISPA_ERR_NULL;
  if (n_jobs < 1 || n_jobs > ISPA_MAX_GROUP || h_in < 1 || h_out < 1) return ISPA_ERR_SHAPE;
  if (h_in % 32 != 0 || h_out % 8 != 0) return ISPA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(h_out) * h_in * 2 > INT32_MAX) return ISPA_ERR_UNSUPPORTED;
  ispa::NtJob nj[ISPA_MAX_GROUP];
  for (int g = 0; g < n_jobs; ++g) {
    const ispa_project_job& j = jobs[g];
    if (j.n < 0) return ISPA_ERR_SHAPE;
    if (j.n > 0 && (!j.x || !j.w || !j.y)) return ISPA_ERR_NULL;
    if (j.n * h_in * 2 > INT32_MAX) return ISPA_ERR_UNSUPPORTED;
    if (j.n > 0 && (!aligned16(j.x) || !aligned16(j.w) || !aligned16(j.y))) return ISPA_ERR_ALIGN;
    nj[g] = ispa::NtJob{static_cast<const uint16_t*>(j.x), static_cast<const uint16_t*>(j.w),
                        static_cast<uint16_t*>(j.y), j.n};
  }
  return hip_status(ispa::launch_nt_gemm256_grouped(nj, n_jobs, h_in, h_out, as_stream(stream)));
}

int ispa_project(const void* x, const void* w, void* y, int64_t n, int h_in, int h_out,
                 void* stream) {
  if (!x || !w || !y) return ISPA_ERR_NULL;
  if (n < 0 || h_in < 1 || h_out < 1) return ISPA_ERR_SHAPE;
  if (h_in % 8 != 0 || h_out % 8 != 0) return ISPA_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return ISPA_ERR_ALIGN;
  if (n == 0) return ISPA_OK;
  return hip_status(ispa::launch_project(static_cast<const uint16_t*>(x),
                                         static_cast<const uint16_t*>(w),
                                         static_cast<uint16_t*>(y), n, h_in, h_out,
                                         as_stream(stream)));
}

}  // extern "C"
