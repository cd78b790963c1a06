// Decomposable attention for CDNA4 (gfx950).
//
// One pass over a chunk's queries produces the local-only result (sink frame
// plus current frames), the history-only result and, by merging their
// log-sum-exp states, the full-history result and D = O_full - O_local.
// ISPA paper ("Towards Memory-Efficient Autoregressive Video Generation via
// Instance-Specific Parametric Absorption"): §3.1 item 1 (A_loc over current
// and sink tokens, A_full over the whole history, collected during warmup),
// §3.4 (decomposable attention on online softmax / LSE states, so both come
// from one attention pass).
//
// Work decomposition: one workgroup = one head x 256 queries, 8 waves of 32
// queries (two per SIMD, one workgroup per CU), so each K/V tile staged in
// LDS serves 256 queries. K/V stream through LDS in 64-key tiles (double
// buffered, one barrier per tile). Per tile and wave:
//   S^T[64 keys x 32 queries] = K Q^T     (16 MFMA 32x32x16, K from LDS,
//                                          Q^T held in registers)
//   online softmax on S^T                 (each lane owns one query, so the
//                                          reductions are in-lane plus one
//                                          exchange with lane^32)
//   O^T[d x 32 queries] += V^T P^T        (16 MFMA, V^T from LDS, P^T taken
//                                          directly from the S^T registers)
// The key order inside V^T is permuted so that the keys a lane holds in its
// S^T registers are exactly the k-slots of the P^T operand.
// The running max is only moved when the tile max exceeds it by more than
// 2^8 (the result is exact either way; it only bounds p <= 256), which keeps
// the O rescale off the common path.

#include <type_traits>

#include "device_common.h"
#include "ispa_internal.h"

namespace ispa {
namespace {

constexpr int kThreads = 512;  // 8 waves
constexpr int kQTile = 256;
constexpr int kKTile = 64;
constexpr float kRescaleThreshold = 8.0f;  // log2 units

// K and V tiles are staged in LDS in their natural [key][d] layout, with
// direct-to-LDS global loads (each wave instruction writes 64 lanes x 16 bytes
// contiguously), swizzled by lds_swz so that both the 16-byte K fragment
// reads and the transposing V reads are free of bank conflicts.
template <int D>
__device__ __forceinline__ int swz(int r) { return lds_swz<D>(r); }

struct Seg {
  const uint16_t* k;
  const uint16_t* v;
  int64_t n;
};

// Direct-to-LDS loads of one 64-key tile of K and V. Each lane's byte offset
// inside a full tile is fixed, so a full tile only moves a uniform base.
// In a tail tile, rows past `valid` re-load the last valid row (in bounds);
// their scores are masked to -inf, so they contribute nothing.
template <int D>
struct TileLoader {
  static constexpr int CPR = D / 8;            // 16-byte chunks per key row
  static constexpr int RPI = 64 / CPR;         // rows per wave instruction
  static constexpr int IPW = kKTile / RPI / (kThreads / 64); // instructions per wave per tensor
  uint32_t off[IPW];                           // bytes, full tile
  int row[IPW];
  int chunk_off;                               // head * D (elements)
  int lds_base;                                // elements

  __device__ void init(int64_t rs, int head, int wave, int lane) {
    const int p = lane % CPR;
    chunk_off = head * D;
    lds_base = wave * IPW * RPI * D;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      row[i] = (wave * IPW + i) * RPI + lane / CPR;
      const int c = p ^ swz<D>(row[i]);
      off[i] = static_cast<uint32_t>((row[i] * rs + head * D + 8 * c) * 2);
    }
  }

  __device__ void issue(const Seg& sg, int64_t row0, int valid, int64_t rs, uint16_t* ks,
                        uint16_t* vs, int lane) const {
    const char* kb = reinterpret_cast<const char*>(sg.k + row0 * rs);
    const char* vb = reinterpret_cast<const char*>(sg.v + row0 * rs);
    if (valid == kKTile) {
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        __builtin_amdgcn_global_load_lds(kb + off[i], ISPA_LDS(void, ks + lds_base + i * RPI * D),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds(vb + off[i], ISPA_LDS(void, vs + lds_base + i * RPI * D),
                                         16, 0, 0);
      }
    } else {
      const int p = lane % CPR;
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int rr = row[i] < valid ? row[i] : valid - 1;
        const int c = p ^ swz<D>(row[i]);
        const int64_t o = (rr * rs + chunk_off + 8 * c) * 2;
        __builtin_amdgcn_global_load_lds(kb + o, ISPA_LDS(void, ks + lds_base + i * RPI * D), 16,
                                         0, 0);
        __builtin_amdgcn_global_load_lds(vb + o, ISPA_LDS(void, vs + lds_base + i * RPI * D), 16,
                                         0, 0);
      }
    }
  }
};

// 16-byte K fragment: key row r, logical chunk c.
template <int D>
__device__ __forceinline__ bf16x8 k_frag(const uint16_t* ks, int r, int c) {
  return *reinterpret_cast<const bf16x8*>(ks + r * D + 8 * (c ^ swz<D>(r)));
}

template <int D>
__device__ __forceinline__ void store_o(uint16_t* out, const f32x16* o, int64_t qi, int64_t rs,
                                        int head, int hf) {
  uint16_t* row = out + qi * rs + head * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * db + 8 * g + 4 * hf;
      uint2 val;
      val.x = pack_bf16x2(o[db][4 * g + 0], o[db][4 * g + 1]);
      val.y = pack_bf16x2(o[db][4 * g + 2], o[db][4 * g + 3]);
      *reinterpret_cast<uint2*>(row + d) = val;
    }
  }
}

template <int D>
__device__ __forceinline__ void store_packed(uint16_t* out, const uint32_t (*o)[8], int64_t qi,
                                             int64_t rs, int head, int hf) {
  uint16_t* row = out + qi * rs + head * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * db + 8 * g + 4 * hf;
      *reinterpret_cast<uint2*>(row + d) = make_uint2(o[db][2 * g], o[db][2 * g + 1]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void attn_decomp_kernel(const AttnParams p) {
  constexpr int TBUF = kKTile * D;   // one K or V tile (elements)
  constexpr int NB = D / 32;
  // Four separate LDS arrays (K and V, two buffers each): every access below
  // names a fixed array, so the compiler can see that the prefetch into one
  // buffer never aliases the reads of the other and needs no early wait.
  __shared__ __attribute__((aligned(16))) uint16_t sk0[TBUF];
  __shared__ __attribute__((aligned(16))) uint16_t sk1[TBUF];
  __shared__ __attribute__((aligned(16))) uint16_t sv0[TBUF];
  __shared__ __attribute__((aligned(16))) uint16_t sv1[TBUF];

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, l32 = lane % 32, hf = lane / 32;
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int head = work / p.n_qtiles;
  const int qt = work % p.n_qtiles;
  const int64_t rs = static_cast<int64_t>(p.n_heads) * D;
  const int64_t qi = static_cast<int64_t>(qt) * kQTile + wave * 32 + l32;
  const bool qvalid = qi < p.n_q;

  // Q^T operand fragments, held for the whole pass.
  bf16x8 qf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    if (qvalid) {
      qf[t] = *reinterpret_cast<const bf16x8*>(p.q + qi * rs + head * D + 16 * t + 8 * hf);
    } else {
      qf[t] = bf16x8{};
    }
  }

  const int nt0 = static_cast<int>((p.n[0] + kKTile - 1) / kKTile);
  const int nt1 = static_cast<int>((p.n[1] + kKTile - 1) / kKTile);
  const int nt2 = static_cast<int>((p.n[2] + kKTile - 1) / kKTile);
  const int n_local_tiles = nt0 + nt1;
  const bool split = p.mode == 0;
  const bool run_hist = !(split && !p.need_hist);
  const int T = n_local_tiles + (run_hist ? nt2 : 0);

  // Flat tile index -> (segment pointers, first row, valid rows). Selected
  // with conditionals so nothing is indexed dynamically (no scratch).
  auto tile_of = [&](int idx, Seg& sg, int64_t& row0, int& valid) {
    const bool s0 = idx < nt0, s1 = !s0 && idx < n_local_tiles;
    const int t = s0 ? idx : (s1 ? idx - nt0 : idx - n_local_tiles);
    sg.k = s0 ? p.k[0] : (s1 ? p.k[1] : p.k[2]);
    sg.v = s0 ? p.v[0] : (s1 ? p.v[1] : p.v[2]);
    sg.n = s0 ? p.n[0] : (s1 ? p.n[1] : p.n[2]);
    row0 = static_cast<int64_t>(t) * kKTile;
    const int64_t rem = sg.n - row0;
    valid = rem < kKTile ? static_cast<int>(rem) : kKTile;
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) oacc[b] = f32x16{};
  // O_local kept as its bf16 output values (the X the statistics see) while
  // the history phase runs: D is then formed against exactly that X.
  uint32_t o_loc[NB][8];
  float lse_loc2 = -INFINITY;


  TileLoader<D> loader;
  loader.init(rs, head, wave, lane);
  {
    Seg sg;
    int valid;
    int64_t row0;
    tile_of(0, sg, row0, valid);
    loader.issue(sg, row0, valid, rs, sk0, sv0, lane);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // One tile; BUF (compile time) selects the LDS buffers it reads, the
  // prefetch of the next tile goes to the other pair.
  auto tile_step = [&](auto buf_c, int idx) {
    constexpr int BUF = decltype(buf_c)::value;
    const uint16_t* ks = BUF ? sk1 : sk0;
    const uint16_t* vs = BUF ? sv1 : sv0;
    uint16_t* nks = BUF ? sk0 : sk1;
    uint16_t* nvs = BUF ? sv0 : sv1;
    Seg sg;
    int valid;
    int64_t row0;
    tile_of(idx, sg, row0, valid);
    const bool has_next = idx + 1 < T;
    if (has_next) {
      Seg s2;
      int v2;
      int64_t r2;
      tile_of(idx + 1, s2, r2, v2);
      loader.issue(s2, r2, v2, rs, nks, nvs, lane);
    }

    // S^T = K Q^T
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const bf16x8 a0 = k_frag<D>(ks, l32, 2 * t + hf);
      const bf16x8 a1 = k_frag<D>(ks, 32 + l32, 2 * t + hf);
      s0 = mfma32x32x16(a0, qf[t], s0);
      s1 = mfma32x32x16(a1, qf[t], s1);
    }

    if (valid < kKTile) {
      // tail tile only: keep this a real branch (the empty volatile asm stops
      // it from being flattened into unconditional selects)
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i / 4) + 4 * hf + (i % 4);
        if (key >= valid) s0[i] = -INFINITY;
        if (key + 32 >= valid) s1[i] = -INFINITY;
      }
    }

    float mx = s0[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s0[i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s1[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mt = mx * p.scale_log2;
    const bool need = mt > m_run + kRescaleThreshold;
    if (__any(need)) {
      const float mnew = need ? mt : m_run;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mnew) : 1.f;
      m_run = mnew;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < NB; ++b) oacc[b] *= alpha;
    }

    // P = 2^(s * scale_log2 - m); the row sum is kept in fp32 (the LSE needs
    // it), P goes to the PV product rounded to bf16.
    bf16x8 pf[4];
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e0 = __builtin_amdgcn_exp2f(fmaf(s0[i], p.scale_log2, -m_run));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(s1[i], p.scale_log2, -m_run));
      lsum += e0 + e1;
      pf[i / 8][i % 8] = static_cast<__bf16>(e0);
      pf[2 + i / 8][i % 8] = static_cast<__bf16>(e1);
    }
    l_run += lsum;

    // O^T += V^T P^T, key step outer so consecutive MFMAs feed independent
    // accumulators
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int db = 0; db < NB; ++db) {
        const bf16x8 a = tr_operand<D>(vs, 16 * st, 32 * db, lane);
        oacc[db] = mfma32x32x16(a, pf[st], oacc[db]);
      }
    }


    if (split && idx == n_local_tiles - 1) {
      const float lt = l_run + __shfl_xor(l_run, 32);
      const float inv = 1.f / lt;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int w = 0; w < 8; ++w)
          o_loc[b][w] = pack_bf16x2(oacc[b][2 * w] * inv, oacc[b][2 * w + 1] * inv);
      }
      lse_loc2 = m_run + __builtin_amdgcn_logf(lt);
      if (qvalid) {
        if (p.o_local) store_packed<D>(p.o_local, o_loc, qi, rs, head, hf);
        if (p.lse_local && hf == 0) p.lse_local[head * p.n_q + qi] = lse_loc2 * kLn2;
      }
      m_run = -INFINITY;
      l_run = 0.f;
#pragma unroll
      for (int b = 0; b < NB; ++b) oacc[b] = f32x16{};
    }
    // the next tile's direct-to-LDS loads (issued at the top) must land
    // before any wave reads them
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  for (int idx = 0; idx < T; idx += 2) {
    tile_step(std::integral_constant<int, 0>{}, idx);
    if (idx + 1 < T) tile_step(std::integral_constant<int, 1>{}, idx + 1);
  }

  if (!qvalid) return;
  if (!split) {
    const float lt = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.f / lt;
#pragma unroll
    for (int b = 0; b < NB; ++b) oacc[b] *= inv;
    if (p.o_full) store_o<D>(p.o_full, oacc, qi, rs, head, hf);
    if (p.lse_full && hf == 0)
      p.lse_full[head * p.n_q + qi] = (m_run + __builtin_amdgcn_logf(lt)) * kLn2;
    return;
  }
  if (!p.need_hist) return;

  // History result (O_H = 0, LSE_H = -inf for an empty history).
  float lse_h2 = -INFINITY;
  if (p.n[2] > 0) {
    const float lt = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.f / lt;
#pragma unroll
    for (int b = 0; b < NB; ++b) oacc[b] *= inv;
    lse_h2 = m_run + __builtin_amdgcn_logf(lt);
  }
  if (p.o_hist) store_o<D>(p.o_hist, oacc, qi, rs, head, hf);
  if (p.lse_hist && hf == 0) p.lse_hist[head * p.n_q + qi] = lse_h2 * kLn2;

  // LSE merge: w_H = 2^(LSE_H - LSE_F), D = w_H (O_H - O_L), O_F = O_L + D.
  float lse_f2 = lse_loc2, w_h = 0.f;
  if (p.n[2] > 0) {
    const float mm = fmaxf(lse_loc2, lse_h2);
    lse_f2 = mm + __builtin_amdgcn_logf(__builtin_amdgcn_exp2f(lse_loc2 - mm) +
                                        __builtin_amdgcn_exp2f(lse_h2 - mm));
    w_h = __builtin_amdgcn_exp2f(lse_h2 - lse_f2);
  }
  f32x16 xl[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      xl[b][2 * w] = __uint_as_float(o_loc[b][w] << 16);
      xl[b][2 * w + 1] = __uint_as_float(o_loc[b][w] & 0xFFFF0000u);
    }
    oacc[b] = (oacc[b] - xl[b]) * w_h;  // D
  }
  if (p.d_out) store_o<D>(p.d_out, oacc, qi, rs, head, hf);
  if (p.o_full) {
#pragma unroll
    for (int b = 0; b < NB; ++b) oacc[b] += xl[b];
    store_o<D>(p.o_full, oacc, qi, rs, head, hf);
  }
  if (p.lse_full && hf == 0) p.lse_full[head * p.n_q + qi] = lse_f2 * kLn2;
}


}  // namespace

hipError_t launch_attn_decomp(AttnParams p, int head_dim, hipStream_t stream) {
  p.n_qtiles = static_cast<int>((p.n_q + kQTile - 1) / kQTile);
  const int blocks = p.n_qtiles * p.n_heads;
  if (blocks == 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_decomp_kernel<128>, dim3(blocks), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_decomp_kernel<64>, dim3(blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

int attn_q_tile_min() { return kQTile; }

}  // namespace ispa
