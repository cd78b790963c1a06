// ISPA streaming session (the ISPA paper: "Towards Memory-Efficient
// Autoregressive Video Generation via Instance-Specific Parametric
// Absorption"). The warmup -> absorption -> streaming life cycle of all
// attention layers over one KV cache, with event-triggered
// recalibration (ISPA paper §3.1 items 1-3, §3.3 including its last
// paragraph). Host-side control only: every step is a call of the C ABI in
// include/ispa.h, enqueued on the caller's stream. Contracts are in
// include/ispa.h.
//
// Phases:
//  warmup  every layer runs the dual-stream attention over sink + history +
//          current (O_local, O_full, D), accumulates G, C, E and projects
//          O_full through the original W; after t_warm chunks the session
//          solves dW (against the original W), scores and selects K layers,
//          writes bf16(W + dW) for them into the active weights, drops their
//          history and prepares their drift state;
//  stream  L-layers attend sink + current through W + dW, F-layers their
//          whole history through W; each L-layer's local output gets a drift
//          score, and when one exceeds the threshold the session re-enters
//          warmup: L-layers get W back and restart their history, and the
//          statistics start over.
// With ISPA_SESSION_W8A8 every projection runs on E4M3 codes of the active
// weights (requantized whenever those change); with ISPA_SESSION_FP8_ATTN
// the streaming phase's attention runs on E4M3 scores, smoothed by a fixed
// per-layer key mean.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <new>
#include <vector>

#include "ispa.h"

namespace {

size_t align_up(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

struct Layout {
  float *G, *C, *E, *dW, *linv;
  void* ridge_ws;
  size_t ridge_bytes;
  void* drift_ws;
  size_t drift_bytes;
  uint16_t *x, *d, *o;
  int *info, *selected;
  double *eps_abs, *eps_rel, *ref, *score;
  // quantized variant (present only with the matching flag)
  uint8_t* wq;           // [n_layers][h, h] E4M3 codes of the active weights
  float* wsc;            // [n_layers][h] their scales
  void* proj_ws;         // ispa_project_w8a8 workspace
  size_t proj_bytes;
  void* attn_ws;         // ispa_attn_decomp_fp8 workspace (largest view)
  size_t attn_bytes;
  uint16_t* mu;          // [n_layers][h] bf16 smoothing vectors
  void* mean_ws;         // ispa_key_mean workspace
  size_t mean_bytes;
  size_t bytes;
};

int64_t drift_sample(const ispa_session_config& c) {
  return (c.n_cur + c.drift_stride - 1) / c.drift_stride;
}

Layout layout(const ispa_session_config& c, void* base) {
  Layout w{};
  const int L = c.n_layers;
  const size_t h = static_cast<size_t>(c.n_heads) * c.head_dim;
  const size_t hh = h * h * L * sizeof(float);
  const size_t act = align_up(static_cast<size_t>(c.n_cur) * h * 2);
  w.ridge_bytes = ispa_ridge_workspace_bytes(L, static_cast<int>(h));
  w.drift_bytes = ispa_drift_workspace_bytes(1, static_cast<int>(h), drift_sample(c));
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t n) {
    char* q = p ? p + off : nullptr;
    off = align_up(off + n);
    return q;
  };
  w.G = reinterpret_cast<float*>(take(hh));
  w.C = reinterpret_cast<float*>(take(hh));
  w.E = reinterpret_cast<float*>(take(hh));
  w.dW = reinterpret_cast<float*>(take(hh));
  w.linv = reinterpret_cast<float*>(take(hh));
  w.ridge_ws = take(w.ridge_bytes);
  w.drift_ws = take(w.drift_bytes);
  w.x = reinterpret_cast<uint16_t*>(take(act));
  w.d = reinterpret_cast<uint16_t*>(take(act));
  w.o = reinterpret_cast<uint16_t*>(take(act));
  w.info = reinterpret_cast<int*>(take(L * sizeof(int)));
  w.selected = reinterpret_cast<int*>(take(L * sizeof(int)));
  w.eps_abs = reinterpret_cast<double*>(take(L * sizeof(double)));
  w.eps_rel = reinterpret_cast<double*>(take(L * sizeof(double)));
  w.ref = reinterpret_cast<double*>(take(L * sizeof(double)));
  w.score = reinterpret_cast<double*>(take(L * sizeof(double)));
  if (c.flags & ISPA_SESSION_W8A8) {
    w.wq = reinterpret_cast<uint8_t*>(take(h * h * L));
    w.wsc = reinterpret_cast<float*>(take(h * L * sizeof(float)));
    w.proj_bytes = ispa_project_w8a8_workspace_bytes(c.n_cur, static_cast<int>(h));
    w.proj_ws = take(w.proj_bytes);
  }
  if (c.flags & ISPA_SESSION_FP8_ATTN) {
    // a view splits sink + history + current into three segments in some
    // way; one segment holding every key plus two of 64 bounds the codes,
    // the per-segment tile padding and the alignment of any split
    w.attn_bytes = ispa_attn_fp8_workspace_bytes(c.n_cur, c.n_sink + c.n_cur + c.hist_capacity,
                                                 64, 64, c.n_heads, c.head_dim);
    w.attn_ws = take(w.attn_bytes);
    w.mu = reinterpret_cast<uint16_t*>(take(h * L * 2));
    w.mean_bytes = ispa_key_mean_workspace_bytes(c.n_heads, c.head_dim);
    w.mean_ws = take(w.mean_bytes);
  }
  w.bytes = off;
  return w;
}

bool valid_config(const ispa_session_config* c) {
  return c->n_layers >= 1 && c->n_heads >= 1 && c->n_cur >= 1 && c->n_sink >= 0 &&
         c->hist_capacity >= 0 && c->t_warm >= 1 && c->k_select >= 0 &&
         c->k_select <= c->n_layers && c->drift_stride >= 1 && c->sm_scale > 0.f &&
         c->lambda >= 0.f && (c->flags & ~(ISPA_SESSION_W8A8 | ISPA_SESSION_FP8_ATTN)) == 0;
}

}  // namespace

struct ispa_session {
  ispa_session_config cfg{};
  ispa_kv_cache* kv = nullptr;
  const uint16_t* wo = nullptr;  // original weights (read only)
  uint16_t* w = nullptr;         // active weights
  Layout ws{};
  int h = 0;
  int64_t hh = 0;
  int phase = ISPA_PHASE_WARMUP;
  int warm_count = 0;
  int64_t chunk = 0;
  int n_calibrations = 0;
  std::vector<int> is_local;     // host copy of the current selection
  std::vector<double> eps_rel;   // host copy of the last errors
  std::vector<double> score;     // host copy of the last drift scores
  std::vector<int> mu_ready;     // smoothing vector of the layer computed
};

namespace {

// E4M3 codes of every layer's active weights (ISPA_SESSION_W8A8).
int requantize(ispa_session* s, void* stream) {
  if (!(s->cfg.flags & ISPA_SESSION_W8A8)) return ISPA_OK;
  return ispa_quantize_fp8(s->w, static_cast<int64_t>(s->cfg.n_layers) * s->h, s->h, s->ws.wq,
                           s->ws.wsc, stream);
}

// y = x W_l^T through the active weights (bf16 or their E4M3 codes).
int project_layer(ispa_session* s, int layer, const void* x, void* y, void* stream) {
  const ispa_session_config& c = s->cfg;
  if (c.flags & ISPA_SESSION_W8A8)
    return ispa_project_w8a8(x, s->ws.wq + layer * s->hh,
                             s->ws.wsc + static_cast<int64_t>(layer) * s->h, y, c.n_cur, s->h,
                             s->h, s->ws.proj_ws, s->ws.proj_bytes, stream);
  return ispa_project(x, s->w + layer * s->hh, y, c.n_cur, s->h, s->h, stream);
}

// Streaming-phase attention of one layer into ws.x: local (sink + current)
// for an L-layer, full for an F-layer; E4M3 scores with ISPA_SESSION_FP8_ATTN.
int stream_attention(ispa_session* s, int layer, const void* q, void* stream) {
  const ispa_session_config& c = s->cfg;
  const bool local = s->is_local[layer] != 0;
  if (!(c.flags & ISPA_SESSION_FP8_ATTN))
    return ispa_kv_attn(s->kv, layer, q, c.n_cur, c.sm_scale, local ? s->ws.x : nullptr, nullptr,
                        nullptr, nullptr, local ? nullptr : s->ws.x, nullptr, nullptr, stream);
  ispa_kv_view v;
  int st = ispa_kv_view_of(s->kv, layer, &v);
  if (st != ISPA_OK) return st;
  uint16_t* mu = s->ws.mu + static_cast<int64_t>(layer) * s->h;
  if (!s->mu_ready[layer]) {
    st = c.n_sink > 0 ? ispa_key_mean(v.k_sink, c.n_sink, nullptr, 0, nullptr, 0, c.n_heads,
                                      c.head_dim, mu, s->ws.mean_ws, s->ws.mean_bytes, stream)
                      : ispa_key_mean(nullptr, 0, v.k_cur, c.n_cur, nullptr, 0, c.n_heads,
                                      c.head_dim, mu, s->ws.mean_ws, s->ws.mean_bytes, stream);
    if (st != ISPA_OK) return st;
    s->mu_ready[layer] = 1;
  }
  if (local && !v.split_ok) return ISPA_ERR_UNSUPPORTED;
  return ispa_attn_decomp_fp8(q, c.n_cur, v.seg_k[0], v.seg_v[0], v.seg_n[0], v.seg_k[1],
                              v.seg_v[1], v.seg_n[1], v.seg_k[2], v.seg_v[2], v.seg_n[2],
                              c.n_heads, c.head_dim, c.sm_scale, mu, local ? s->ws.x : nullptr,
                              nullptr, nullptr, nullptr, local ? nullptr : s->ws.x, nullptr,
                              nullptr, s->ws.attn_ws, s->ws.attn_bytes, stream);
}

}  // namespace

extern "C" {

size_t ispa_session_workspace_bytes(const ispa_session_config* cfg) {
  if (!cfg || !valid_config(cfg)) return 0;
  return layout(*cfg, nullptr).bytes;
}

int ispa_session_create(const ispa_session_config* cfg, const void* wo, void* w_active,
                        void* workspace, size_t ws_bytes, void* stream, ispa_session** out) {
  if (!out) return ISPA_ERR_NULL;
  *out = nullptr;
  if (!cfg || !wo || !w_active || !workspace) return ISPA_ERR_NULL;
  if (!valid_config(cfg)) return ISPA_ERR_SHAPE;
  if (cfg->head_dim != 64 && cfg->head_dim != 128) return ISPA_ERR_UNSUPPORTED;
  if ((cfg->flags & ISPA_SESSION_FP8_ATTN) && cfg->head_dim != 128) return ISPA_ERR_UNSUPPORTED;
  if ((cfg->flags & ISPA_SESSION_W8A8) && (cfg->n_heads * cfg->head_dim) % 64 != 0)
    return ISPA_ERR_UNSUPPORTED;
  if (ws_bytes < layout(*cfg, nullptr).bytes) return ISPA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(wo) | reinterpret_cast<uintptr_t>(w_active) |
       reinterpret_cast<uintptr_t>(workspace)) & 15u)
    return ISPA_ERR_ALIGN;
  ispa_session* s = new (std::nothrow) ispa_session();
  if (!s) return ISPA_ERR_HIP;
  s->cfg = *cfg;
  s->h = cfg->n_heads * cfg->head_dim;
  s->hh = static_cast<int64_t>(s->h) * s->h;
  s->wo = static_cast<const uint16_t*>(wo);
  s->w = static_cast<uint16_t*>(w_active);
  s->ws = layout(*cfg, workspace);
  s->is_local.assign(cfg->n_layers, 0);
  s->eps_rel.assign(cfg->n_layers, 0.0);
  s->score.assign(cfg->n_layers, 0.0);
  s->mu_ready.assign(cfg->n_layers, 0);
  int st = ispa_kv_create(cfg->n_layers, cfg->n_heads, cfg->head_dim, cfg->n_sink, cfg->n_cur,
                          cfg->hist_capacity, &s->kv);
  if (st != ISPA_OK) {
    delete s;
    return st;
  }
  // the active weights start as the original ones
  if (hipMemcpyAsync(s->w, s->wo, static_cast<size_t>(s->hh) * cfg->n_layers * 2,
                     hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream)) != hipSuccess) {
    ispa_kv_destroy(s->kv);
    delete s;
    return ISPA_ERR_HIP;
  }
  if ((st = requantize(s, stream)) != ISPA_OK) {
    ispa_kv_destroy(s->kv);
    delete s;
    return st;
  }
  *out = s;
  return ISPA_OK;
}

int ispa_session_destroy(ispa_session* s) {
  if (!s) return ISPA_ERR_NULL;
  const int st = ispa_kv_destroy(s->kv);
  delete s;
  return st;
}

ispa_kv_cache* ispa_session_cache(ispa_session* s) { return s ? s->kv : nullptr; }

int ispa_session_layer(ispa_session* s, int layer, const void* q, void* y, void* stream) {
  if (!s || !q || !y) return ISPA_ERR_NULL;
  const ispa_session_config& c = s->cfg;
  if (layer < 0 || layer >= c.n_layers) return ISPA_ERR_SHAPE;
  if (s->phase == ISPA_PHASE_WARMUP) {
    // dual stream: X = O_local and D into the statistics, O_full projected
    int st = ispa_kv_attn(s->kv, layer, q, c.n_cur, c.sm_scale, s->ws.x, nullptr, nullptr,
                          nullptr, s->ws.o, nullptr, s->ws.d, stream);
    if (st != ISPA_OK) return st;
    st = ispa_gram_accumulate(s->ws.x, s->ws.d, c.n_cur, s->h, 1, s->ws.G + layer * s->hh,
                              s->ws.C + layer * s->hh, s->ws.E + layer * s->hh,
                              s->warm_count == 0 ? 1 : 0, stream);
    if (st != ISPA_OK) return st;
    return project_layer(s, layer, s->ws.o, y, stream);
  }
  int st = stream_attention(s, layer, q, stream);
  if (st == ISPA_OK) st = project_layer(s, layer, s->ws.x, y, stream);
  if (st != ISPA_OK || !s->is_local[layer] || c.drift_threshold <= 0.0) return st;
  return ispa_drift_score(1, s->h, s->ws.linv + layer * s->hh, s->ws.ref + layer, s->ws.x,
                          c.n_cur, c.drift_stride, s->ws.score + layer, s->ws.drift_ws,
                          s->ws.drift_bytes, stream);
}

int ispa_session_layer_grouped(ispa_session* const* s, int n, int layer, const void* const* q,
                               void* const* y, void* stream) {
  if (!s || !q || !y) return ISPA_ERR_NULL;
  if (n < 1 || n > ISPA_MAX_GROUP) return ISPA_ERR_SHAPE;
  for (int g = 0; g < n; ++g) {
    if (!s[g] || !q[g] || !y[g]) return ISPA_ERR_NULL;
    const ispa_session_config& a = s[g]->cfg;
    const ispa_session_config& b = s[0]->cfg;
    if (a.n_heads != b.n_heads || a.head_dim != b.head_dim || a.n_cur != b.n_cur ||
        layer < 0 || layer >= a.n_layers)
      return ISPA_ERR_SHAPE;
  }
  const ispa_session_config& c0 = s[0]->cfg;
  ispa_attn_job jobs[ISPA_MAX_GROUP] = {};
  ispa_project_job proj[ISPA_MAX_GROUP] = {};
  int grouped[ISPA_MAX_GROUP];
  int m = 0;
  for (int g = 0; g < n; ++g) {
    ispa_session* sg = s[g];
    if (sg->phase != ISPA_PHASE_STREAM || sg->cfg.flags != 0) {
      const int st = ispa_session_layer(sg, layer, q[g], y[g], stream);
      if (st != ISPA_OK) return st;
      continue;
    }
    ispa_kv_view v;
    int st = ispa_kv_view_of(sg->kv, layer, &v);
    if (st != ISPA_OK) return st;
    const bool local = sg->is_local[layer] != 0;
    if (local && !v.split_ok) return ISPA_ERR_UNSUPPORTED;
    ispa_attn_job& j = jobs[m];
    j.q = q[g];
    j.n_q = sg->cfg.n_cur;
    j.k_sink = v.seg_k[0];
    j.v_sink = v.seg_v[0];
    j.n_sink = v.seg_n[0];
    j.k_cur = v.seg_k[1];
    j.v_cur = v.seg_v[1];
    j.n_cur = v.seg_n[1];
    j.k_hist = v.seg_k[2];
    j.v_hist = v.seg_v[2];
    j.n_hist = v.seg_n[2];
    (local ? j.o_local : j.o_full) = sg->ws.x;
    proj[m] = ispa_project_job{sg->ws.x, sg->w + layer * sg->hh, y[g], sg->cfg.n_cur};
    grouped[m++] = g;
  }
  if (m == 0) return ISPA_OK;
  // the sessions share the softmax scale only if their configurations do
  bool same_scale = true;
  for (int k = 1; k < m; ++k)
    same_scale &= s[grouped[k]]->cfg.sm_scale == s[grouped[0]]->cfg.sm_scale;
  int st = ISPA_OK;
  if (same_scale) {
    st = ispa_attn_decomp_grouped(jobs, m, c0.n_heads, c0.head_dim, s[grouped[0]]->cfg.sm_scale,
                                  stream);
  } else {
    for (int k = 0; k < m && st == ISPA_OK; ++k)
      st = ispa_attn_decomp_grouped(&jobs[k], 1, c0.n_heads, c0.head_dim,
                                    s[grouped[k]]->cfg.sm_scale, stream);
  }
  if (st != ISPA_OK) return st;
  const int h = s[grouped[0]]->h;
  if (h % 32 == 0) {
    st = ispa_project_grouped(proj, m, h, h, stream);
  } else {
    for (int k = 0; k < m && st == ISPA_OK; ++k)
      st = ispa_project(proj[k].x, proj[k].w, proj[k].y, proj[k].n, h, h, stream);
  }
  if (st != ISPA_OK) return st;
  for (int k = 0; k < m; ++k) {
    ispa_session* sg = s[grouped[k]];
    const ispa_session_config& c = sg->cfg;
    if (!sg->is_local[layer] || c.drift_threshold <= 0.0) continue;
    st = ispa_drift_score(1, sg->h, sg->ws.linv + layer * sg->hh, sg->ws.ref + layer, sg->ws.x,
                          c.n_cur, c.drift_stride, sg->ws.score + layer, sg->ws.drift_ws,
                          sg->ws.drift_bytes, stream);
    if (st != ISPA_OK) return st;
  }
  return ISPA_OK;
}

int ispa_session_end_chunk(ispa_session* s, void* stream, int* event) {
  if (!s) return ISPA_ERR_NULL;
  const ispa_session_config& c = s->cfg;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const int L = c.n_layers;
  if (event) *event = ISPA_EVENT_NONE;
  int st = ispa_kv_advance(s->kv);
  if (st != ISPA_OK) return st;
  ++s->chunk;
  if (s->phase == ISPA_PHASE_WARMUP) {
    if (++s->warm_count < c.t_warm) return ISPA_OK;
    // transition: solve against the original W, score, select, update
    st = ispa_ridge_solve(L, s->h, s->ws.G, s->ws.C, s->wo, c.lambda, s->ws.dW, s->ws.info,
                          s->ws.ridge_ws, s->ws.ridge_bytes, stream);
    // the drift reference from the ridge's own factor of G + lambda I, before
    // the score reuses its storage
    if (st == ISPA_OK && c.drift_threshold > 0.0)
      st = ispa_drift_prepare_factored(L, s->h, c.lambda, c.n_cur * c.t_warm, s->ws.linv,
                                       s->ws.ref, s->ws.ridge_ws, s->ws.ridge_bytes, stream);
    if (st == ISPA_OK)
      st = ispa_layer_score(L, s->h, s->ws.G, s->ws.C, s->ws.E, s->wo, s->ws.dW, c.lambda,
                            s->ws.info, c.k_select, s->ws.ridge_ws, s->ws.ridge_bytes,
                            s->ws.eps_abs, s->ws.eps_rel, s->ws.selected, stream);
    if (st == ISPA_OK && hipMemcpyAsync(s->w, s->wo, static_cast<size_t>(s->hh) * L * 2,
                                        hipMemcpyDeviceToDevice, hs) != hipSuccess)
      st = ISPA_ERR_HIP;
    if (st == ISPA_OK) st = ispa_apply_dW(L, s->h, s->ws.selected, s->ws.dW, s->w, stream);
    if (st == ISPA_OK) st = requantize(s, stream);
    if (st != ISPA_OK) return st;
    // which layers turn local is a host decision: their history is freed
    std::vector<int> sel(L);
    if (hipMemcpyAsync(sel.data(), s->ws.selected, L * sizeof(int), hipMemcpyDeviceToHost, hs) !=
            hipSuccess ||
        hipMemcpyAsync(s->eps_rel.data(), s->ws.eps_rel, L * sizeof(double),
                       hipMemcpyDeviceToHost, hs) != hipSuccess ||
        hipStreamSynchronize(hs) != hipSuccess)
      return ISPA_ERR_HIP;
    for (int l = 0; l < L; ++l) {
      s->is_local[l] = sel[l] ? 1 : 0;
      s->score[l] = 0.0;
      if (sel[l] && (st = ispa_kv_evict_history(s->kv, l, stream)) != ISPA_OK) return st;
    }
    s->phase = ISPA_PHASE_STREAM;
    ++s->n_calibrations;
    if (event) *event = ISPA_EVENT_ABSORBED;
    return ISPA_OK;
  }
  if (c.drift_threshold <= 0.0) return ISPA_OK;
  // drift check of the L-layers of the chunk just run
  if (hipMemcpyAsync(s->score.data(), s->ws.score, L * sizeof(double), hipMemcpyDeviceToHost,
                     hs) != hipSuccess ||
      hipStreamSynchronize(hs) != hipSuccess)
    return ISPA_ERR_HIP;
  bool trigger = false;
  for (int l = 0; l < L; ++l) {
    if (!s->is_local[l]) {
      s->score[l] = 0.0;
      continue;
    }
    // NaN (a failed factor) counts as drift
    if (!(s->score[l] <= c.drift_threshold)) trigger = true;
  }
  if (!trigger) return ISPA_OK;
  // recalibration: L-layers get W back and restart their history; the
  // statistics start over with the next chunk
  for (int l = 0; l < L; ++l)
    if (s->is_local[l] && (st = ispa_kv_restore_history(s->kv, l)) != ISPA_OK) return st;
  if (hipMemcpyAsync(s->w, s->wo, static_cast<size_t>(s->hh) * L * 2, hipMemcpyDeviceToDevice,
                     hs) != hipSuccess)
    return ISPA_ERR_HIP;
  if ((st = requantize(s, stream)) != ISPA_OK) return st;
  std::fill(s->is_local.begin(), s->is_local.end(), 0);
  s->phase = ISPA_PHASE_WARMUP;
  s->warm_count = 0;
  if (event) *event = ISPA_EVENT_RECALIBRATE;
  return ISPA_OK;
}

int ispa_session_query(const ispa_session* s, ispa_session_state* out, int* is_local,
                       double* eps_rel, double* drift) {
  if (!s || !out) return ISPA_ERR_NULL;
  out->phase = s->phase;
  out->warm_count = s->warm_count;
  out->n_calibrations = s->n_calibrations;
  out->chunk = s->chunk;
  const int L = s->cfg.n_layers;
  for (int l = 0; l < L; ++l) {
    if (is_local) is_local[l] = s->is_local[l];
    if (eps_rel) eps_rel[l] = s->eps_rel[l];
    if (drift) drift[l] = s->score[l];
  }
  return ISPA_OK;
}

}  // extern "C"
