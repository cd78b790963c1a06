// Streaming KV cache of the attention layers and the per-layer streaming
// step (ISPA paper §3.1 item 3 and §3.3: after the transition the K selected
// layers attend the sink and current tokens only, through W + dW, and their
// history KV is dropped for good; the other layers keep attending their whole
// history through W). Contracts are in include/ispa.h.
//
// Layout. Each layer's K and V live in one reserved virtual address range
// each, as rows of [n_heads, head_dim] bf16:
//   [ sink (n_sink rows) | slot 0 | slot 1 | ... | slot S-1 ],  slot = n_cur rows.
// Chunk c of a full-history layer is written to slot c mod S and its history
// is every other filled slot, so a capacity of S-1 chunks keeps the S-1 most
// recent ones. Until the ring wraps the history is slots [0, c), directly
// after the sink, and the current chunk follows it: the attention reads three
// plain segments (sink, current, history) and the chunk's K/V never move.
// Softmax attention does not depend on the order of the keys, so a wrapped
// ring (slots out of time order) still gives the full-history output.
//
// Memory. Physical memory is mapped page by page as slots are first used,
// so a layer holds what its history needs rather than its capacity; a layer
// that turns local-only releases every page past those of the sink and slot
// 0. Mapping is a host call that does not wait for the GPU; unmapping waits
// for the caller's stream first.

#include <hip/hip_runtime.h>

#include <stdio.h>

#include <new>
#include <vector>

#include "ispa.h"
#include "ispa_internal.h"

namespace {

struct Piece {
  size_t off;
  size_t size;
  hipMemGenericAllocationHandle_t handle;
};

// One reserved range with the prefix [0, mapped) backed by physical memory.
struct Range {
  char* base = nullptr;
  size_t reserved = 0;
  size_t mapped = 0;
  std::vector<Piece> pieces;
};

struct LayerKV {
  Range k, v;
  int64_t chunk = 0;        // current chunk, counted from the first one the layer kept
  bool local_only = false;
};

size_t round_up(size_t v, size_t g) { return (v + g - 1) / g * g; }

// Memory is mapped in pages of one size per cache, each its own allocation,
// mapping and access grant, naturally aligned in the range: the smallest
// power of two that holds one chunk's rows, at least 2 MiB (the large-page
// size) and at most 256 MiB. A full-history layer then maps about one page
// per chunk, which keeps the number of live mappings (each a process
// mapping of its own) in the thousands for 14B-sized histories, where 2 MiB
// pages would need tens of thousands; the waste is under one page per range.
constexpr size_t kPageMin = size_t{2} << 20;
constexpr size_t kPageMax = size_t{256} << 20;

size_t page_size(size_t chunk_bytes, size_t gran) {
  size_t p = kPageMin;
  while (p < chunk_bytes && p < kPageMax) p <<= 1;
  return round_up(p > gran ? p : gran, gran);
}

// Text of the last failed HIP call (per cache; per thread for creation).
struct ErrText {
  char text[224] = {0};
  void set(const char* call, hipError_t e, size_t off, size_t size) {
    snprintf(text, sizeof(text), "%s(offset %zu, size %zu): %s (%d)", call, off, size,
             hipGetErrorString(e), static_cast<int>(e));
  }
};
thread_local ErrText g_create_error;

hipMemAllocationProp device_prop(int device) {
  hipMemAllocationProp prop{};
  prop.type = hipMemAllocationTypePinned;
  prop.location.type = hipMemLocationTypeDevice;
  prop.location.id = device;
  return prop;
}

// Back one page at offset r.mapped.
hipError_t map_page(Range& r, size_t size, int device, ErrText& err) {
  const size_t off = r.mapped;
  const hipMemAllocationProp prop = device_prop(device);
  hipMemGenericAllocationHandle_t h{};
  hipError_t e = hipMemCreate(&h, size, &prop, 0);
  if (e != hipSuccess) {
    err.set("hipMemCreate", e, off, size);
    return e;
  }
  e = hipMemMap(r.base + off, size, 0, h, 0);
  if (e != hipSuccess) {
    err.set("hipMemMap", e, off, size);
    (void)hipMemRelease(h);
    return e;
  }
  hipMemAccessDesc acc{};
  acc.location = prop.location;
  acc.flags = hipMemAccessFlagsProtReadWrite;
  e = hipMemSetAccess(r.base + off, size, &acc, 1);
  if (e != hipSuccess) {
    err.set("hipMemSetAccess", e, off, size);
    (void)hipMemUnmap(r.base + off, size);
    (void)hipMemRelease(h);
    return e;
  }
  r.pieces.push_back({off, size, h});
  r.mapped = off + size;
  return hipSuccess;
}

// Back [0, need) (rounded up to whole pages, at most the reservation).
hipError_t map_prefix(Range& r, size_t need, size_t piece, int device, ErrText& err) {
  need = round_up(need, piece);
  if (need > r.reserved) need = r.reserved;
  while (r.mapped < need) {
    const hipError_t e = map_page(r, piece, device, err);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Unmap and free every piece past the first `keep`.
hipError_t unmap_tail(Range& r, size_t keep, ErrText& err) {
  hipError_t first = hipSuccess;
  while (r.pieces.size() > keep) {
    const Piece p = r.pieces.back();
    r.pieces.pop_back();
    hipError_t e = hipMemUnmap(r.base + p.off, p.size);
    if (e != hipSuccess) {
      err.set("hipMemUnmap", e, p.off, p.size);
    } else {
      e = hipMemRelease(p.handle);
      if (e != hipSuccess) err.set("hipMemRelease", e, p.off, p.size);
    }
    if (e != hipSuccess && first == hipSuccess) first = e;
    r.mapped = p.off;
  }
  return first;
}

void free_range(Range& r, ErrText& err) {
  (void)unmap_tail(r, 0, err);
  if (r.base) (void)hipMemAddressFree(r.base, r.reserved);
  r.base = nullptr;
  r.reserved = r.mapped = 0;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

struct ispa_kv_cache {
  int n_layers = 0, n_heads = 0, head_dim = 0, device = 0;
  int64_t n_sink = 0, n_cur = 0, n_slots = 0;
  size_t row_bytes = 0, piece = 0;
  std::vector<LayerKV> layers;
  ErrText err;

  size_t rows_bytes(int64_t rows) const { return static_cast<size_t>(rows) * row_bytes; }
  size_t slot_row(int64_t s) const { return static_cast<size_t>(n_sink + s * n_cur); }
  // Rows that must be backed while slot s is current (sink + slots 0..s).
  size_t need_bytes(int64_t s) const { return rows_bytes(n_sink + (s + 1) * n_cur); }
};

namespace {

bool valid_layer(const ispa_kv_cache* c, int layer) {
  return c && layer >= 0 && layer < c->n_layers;
}

void fill_view(const ispa_kv_cache* c, int layer, ispa_kv_view* v) {
  const LayerKV& L = c->layers[layer];
  char* kb = L.k.base;
  char* vb = L.v.base;
  const int64_t S = c->n_slots;
  const int64_t s = L.local_only ? 0 : L.chunk % S;
  const int64_t hist_chunks = L.local_only ? 0 : (L.chunk < S ? L.chunk : S - 1);
  const bool wrapped = !L.local_only && L.chunk >= S;
  *v = ispa_kv_view{};
  v->k_sink = kb;
  v->v_sink = vb;
  v->k_cur = kb + c->rows_bytes(c->slot_row(s));
  v->v_cur = vb + c->rows_bytes(c->slot_row(s));
  v->n_hist = hist_chunks * c->n_cur;
  v->local_only = L.local_only ? 1 : 0;
  v->split_ok = (!wrapped || s == 0) ? 1 : 0;
  v->seg_k[1] = v->k_cur;
  v->seg_v[1] = v->v_cur;
  v->seg_n[1] = c->n_cur;
  if (!wrapped) {
    // sink | history (slots 0 .. s-1) | current (slot s)
    v->seg_k[0] = kb;
    v->seg_v[0] = vb;
    v->seg_n[0] = c->n_sink;
    v->seg_k[2] = kb + c->rows_bytes(c->n_sink);
    v->seg_v[2] = vb + c->rows_bytes(c->n_sink);
    v->seg_n[2] = v->n_hist;
  } else {
    // sink + slots [0, s) | current (slot s) | slots (s, S)
    v->seg_k[0] = kb;
    v->seg_v[0] = vb;
    v->seg_n[0] = c->n_sink + s * c->n_cur;
    v->seg_k[2] = kb + c->rows_bytes(c->slot_row(s + 1));
    v->seg_v[2] = vb + c->rows_bytes(c->slot_row(s + 1));
    v->seg_n[2] = (S - 1 - s) * c->n_cur;
  }
  for (int i = 0; i < 3; ++i)
    if (v->seg_n[i] == 0) v->seg_k[i] = v->seg_v[i] = nullptr;
}

}  // namespace

extern "C" {

int ispa_kv_create(int n_layers, int n_heads, int head_dim, int64_t n_sink, int64_t n_cur,
                   int64_t hist_capacity, ispa_kv_cache** out) {
  if (!out) return ISPA_ERR_NULL;
  *out = nullptr;
  if (n_layers < 1 || n_heads < 1 || n_sink < 0 || n_cur < 1 || hist_capacity < 0 ||
      hist_capacity % n_cur != 0)
    return ISPA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return ISPA_ERR_UNSUPPORTED;
  const size_t row = static_cast<size_t>(n_heads) * head_dim * 2;
  const int64_t n_slots = hist_capacity / n_cur + 1;
  // reservation of one range, with overflow checks (rows * row bytes < 2^62)
  const int64_t rows = n_sink + n_slots * n_cur;
  if (n_slots > (INT64_MAX / 4) / n_cur || rows > (INT64_MAX / 4) / static_cast<int64_t>(row))
    return ISPA_ERR_SHAPE;

  int device = 0, vmm = 0;
  if (hipGetDevice(&device) != hipSuccess) return ISPA_ERR_HIP;
  if (hipDeviceGetAttribute(&vmm, hipDeviceAttributeVirtualMemoryManagementSupported, device) !=
      hipSuccess)
    return ISPA_ERR_HIP;
  if (!vmm) return ISPA_ERR_UNSUPPORTED;
  size_t gran = 0;
  const hipMemAllocationProp prop = device_prop(device);
  const hipError_t ge =
      hipMemGetAllocationGranularity(&gran, &prop, hipMemAllocationGranularityRecommended);
  if (ge != hipSuccess || gran == 0) {
    g_create_error.set("hipMemGetAllocationGranularity", ge, 0, gran);
    return ISPA_ERR_HIP;
  }
  const size_t piece = page_size(static_cast<size_t>(n_cur) * row, gran);

  ispa_kv_cache* c = new (std::nothrow) ispa_kv_cache();
  if (!c) return ISPA_ERR_HIP;
  c->n_layers = n_layers;
  c->n_heads = n_heads;
  c->head_dim = head_dim;
  c->device = device;
  c->n_sink = n_sink;
  c->n_cur = n_cur;
  c->n_slots = n_slots;
  c->row_bytes = row;
  c->piece = piece;
  c->layers.resize(n_layers);
  const size_t bytes = round_up(static_cast<size_t>(rows) * row, piece);
  for (LayerKV& L : c->layers) {
    for (Range* r : {&L.k, &L.v}) {
      void* base = nullptr;
      const hipError_t re = hipMemAddressReserve(&base, bytes, piece, nullptr, 0);
      if (re != hipSuccess) {
        g_create_error.set("hipMemAddressReserve", re, 0, bytes);
        ispa_kv_destroy(c);
        return ISPA_ERR_HIP;
      }
      r->base = static_cast<char*>(base);
      r->reserved = bytes;
      if (map_prefix(*r, c->need_bytes(0), piece, device, g_create_error) != hipSuccess) {
        ispa_kv_destroy(c);
        return ISPA_ERR_HIP;
      }
    }
  }
  *out = c;
  return ISPA_OK;
}

int ispa_kv_destroy(ispa_kv_cache* cache) {
  if (!cache) return ISPA_ERR_NULL;
  // pending kernels may still read the ranges
  const hipError_t e = hipDeviceSynchronize();
  for (LayerKV& L : cache->layers) {
    free_range(L.k, cache->err);
    free_range(L.v, cache->err);
  }
  delete cache;
  return e == hipSuccess ? ISPA_OK : ISPA_ERR_HIP;
}

int ispa_kv_view_of(const ispa_kv_cache* cache, int layer, ispa_kv_view* view) {
  if (!cache || !view) return ISPA_ERR_NULL;
  if (!valid_layer(cache, layer)) return ISPA_ERR_SHAPE;
  fill_view(cache, layer, view);
  return ISPA_OK;
}

int ispa_kv_write(ispa_kv_cache* cache, int layer, int which, const void* k, const void* v,
                  void* stream) {
  if (!cache || !k || !v) return ISPA_ERR_NULL;
  if (!valid_layer(cache, layer) || (which != ISPA_KV_CURRENT && which != ISPA_KV_SINK))
    return ISPA_ERR_SHAPE;
  ispa_kv_view view;
  fill_view(cache, layer, &view);
  const bool cur = which == ISPA_KV_CURRENT;
  const size_t bytes = cache->rows_bytes(cur ? cache->n_cur : cache->n_sink);
  if (bytes == 0) return ISPA_OK;
  void* dk = cur ? view.k_cur : view.k_sink;
  void* dv = cur ? view.v_cur : view.v_sink;
  const hipStream_t s = as_stream(stream);
  if (hipMemcpyAsync(dk, k, bytes, hipMemcpyDeviceToDevice, s) != hipSuccess ||
      hipMemcpyAsync(dv, v, bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return ISPA_ERR_HIP;
  return ISPA_OK;
}

int ispa_kv_advance(ispa_kv_cache* cache) {
  if (!cache) return ISPA_ERR_NULL;
  // back the next slot of every full-history layer first, then move on, so
  // that a failed mapping leaves every layer where it was
  for (LayerKV& L : cache->layers) {
    if (L.local_only) continue;
    const int64_t s = (L.chunk + 1) % cache->n_slots;
    const size_t need = cache->need_bytes(s);
    if (map_prefix(L.k, need, cache->piece, cache->device, cache->err) != hipSuccess ||
        map_prefix(L.v, need, cache->piece, cache->device, cache->err) != hipSuccess)
      return ISPA_ERR_HIP;
  }
  for (LayerKV& L : cache->layers)
    if (!L.local_only) ++L.chunk;
  return ISPA_OK;
}

int ispa_kv_evict_history(ispa_kv_cache* cache, int layer, void* stream) {
  if (!cache) return ISPA_ERR_NULL;
  if (!valid_layer(cache, layer)) return ISPA_ERR_SHAPE;
  LayerKV& L = cache->layers[layer];
  if (L.local_only) return ISPA_OK;
  // work already enqueued on the stream may still read the history
  if (hipStreamSynchronize(as_stream(stream)) != hipSuccess) return ISPA_ERR_HIP;
  L.local_only = true;
  L.chunk = 0;
  // keep the pages of the sink and slot 0
  const size_t keep = round_up(cache->need_bytes(0), cache->piece) / cache->piece;
  const hipError_t ek = unmap_tail(L.k, keep, cache->err);
  const hipError_t ev = unmap_tail(L.v, keep, cache->err);
  return (ek == hipSuccess && ev == hipSuccess) ? ISPA_OK : ISPA_ERR_HIP;
}

int ispa_kv_restore_history(ispa_kv_cache* cache, int layer) {
  if (!cache) return ISPA_ERR_NULL;
  if (!valid_layer(cache, layer)) return ISPA_ERR_SHAPE;
  LayerKV& L = cache->layers[layer];
  // an L-layer writes slot 0: as a full-history layer at chunk 0 that slot is
  // its current one and the history is empty
  if (L.local_only) {
    L.local_only = false;
    L.chunk = 0;
  }
  return ISPA_OK;
}

const char* ispa_kv_last_error(const ispa_kv_cache* cache) {
  return cache ? cache->err.text : g_create_error.text;
}

int64_t ispa_kv_resident_bytes(const ispa_kv_cache* cache) {
  if (!cache) return -1;
  int64_t total = 0;
  for (const LayerKV& L : cache->layers)
    total += static_cast<int64_t>(L.k.mapped + L.v.mapped);
  return total;
}

int ispa_kv_attn(const ispa_kv_cache* cache, int layer, const void* q, int64_t n_q,
                 float sm_scale, void* o_local, float* lse_local, void* o_hist, float* lse_hist,
                 void* o_full, float* lse_full, void* d_out, void* stream) {
  if (!cache) return ISPA_ERR_NULL;
  if (!valid_layer(cache, layer)) return ISPA_ERR_SHAPE;
  ispa_kv_view v;
  fill_view(cache, layer, &v);
  const bool split = o_local || lse_local || o_hist || lse_hist || d_out;
  if (split && !v.split_ok) {
    // a wrapped ring: sink | slots [0, s) | current (slot s) | slots (s, S);
    // the history is slots (s, S) then slots [0, s), two pieces
    const LayerKV& L = cache->layers[layer];
    const int64_t s = L.chunk % cache->n_slots;
    char* kb = L.k.base;
    char* vb = L.v.base;
    const int64_t first = cache->rows_bytes(cache->n_sink);
    return ispa::attn_decomp_two_piece_history(
        q, n_q, v.k_sink, v.v_sink, cache->n_sink, v.k_cur, v.v_cur, cache->n_cur, v.seg_k[2],
        v.seg_v[2], v.seg_n[2], kb + first, vb + first, s * cache->n_cur, cache->n_heads,
        cache->head_dim, sm_scale, o_local, lse_local, o_hist, lse_hist, o_full, lse_full, d_out,
        stream);
  }
  return ispa_attn_decomp(q, n_q, v.seg_k[0], v.seg_v[0], v.seg_n[0], v.seg_k[1], v.seg_v[1],
                          v.seg_n[1], v.seg_k[2], v.seg_v[2], v.seg_n[2], cache->n_heads,
                          cache->head_dim, sm_scale, o_local, lse_local, o_hist, lse_hist, o_full,
                          lse_full, d_out, stream);
}

int ispa_kv_layer_forward(const ispa_kv_cache* cache, int layer, const void* q, int64_t n_q,
                          float sm_scale, const void* wo, void* o_tmp, void* y, void* stream) {
  if (!cache || !wo || !o_tmp || !y) return ISPA_ERR_NULL;
  if (!valid_layer(cache, layer)) return ISPA_ERR_SHAPE;
  const int h = cache->n_heads * cache->head_dim;
  // validate the projection before anything is enqueued
  const int pst = ispa_project(o_tmp, wo, y, 0, h, h, stream);
  if (pst != ISPA_OK) return pst;
  const bool local = cache->layers[layer].local_only;
  const int st = ispa_kv_attn(cache, layer, q, n_q, sm_scale, local ? o_tmp : nullptr, nullptr,
                              nullptr, nullptr, local ? nullptr : o_tmp, nullptr, nullptr, stream);
  if (st != ISPA_OK) return st;
  return ispa_project(o_tmp, wo, y, n_q, h, h, stream);
}

}  // extern "C"
