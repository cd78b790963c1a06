// Decomposable attention for CDNA4 (gfx950).
//
// One pass over a chunk's queries produces the local-only result (sink frame
// plus current frames), the history-only result and, by merging their
// log-sum-exp states, the full-history result and D = O_full - O_local. The
// history may come in two pieces (the two ranges of a ring buffer that has
// wrapped); attention does not depend on the order of its keys.
// ISPA paper ("Towards Memory-Efficient Autoregressive Video Generation via
// Instance-Specific Parametric Absorption"): §3.1 item 1 (A_loc over current
// and sink tokens, A_full over the whole history, collected during warmup),
// §3.4 (decomposable attention on online softmax / LSE states, so both come
// from one attention pass).
//
// Work decomposition: one workgroup = one head x 256 queries, 8 waves in 4
// pairs of 64 queries (two 32-query blocks). In a pair the S-wave computes
// the scores and the online softmax, the O-wave accumulates the output one
// tile behind it; both run on one SIMD. K/V stream through LDS in 64-key
// tiles (double buffered, one barrier per tile); the O-wave issues every
// tile load (V of its own tile, K two tiles ahead), so the S-wave, which
// carries the vector work, never waits on the memory pipeline. Per tile and
// pair:
//   S-wave: the online softmax of tile j on S^T (each lane owns one query per
//           block: in-lane reductions plus one exchange between the lane
//           halves), P^T to LDS in the MFMA operand layout with the rescale
//           factors of any move of the running max, interleaved slice by
//           slice with S^T[64 keys x 64 queries] = K Q^T of tile j+1
//           (32 MFMA 32x32x16, K from LDS with 16-byte reads, Q^T in
//           registers), so the vector work runs while the matrix cores are
//           busy.
//   O-wave: O^T[d x 64 queries] = alpha O^T + V^T P^T of tile j-1 (32 MFMA,
//           V^T by transposing LDS reads several MFMAs ahead, P^T by 16-byte
//           reads), then the loads of the next tiles, issued after P V so
//           that their LDS writes do not hold up its operand reads.
// Each K and V fragment read from LDS feeds two MFMAs (both query blocks).
// The key order inside V^T is permuted so that the keys a lane holds in its
// S^T registers are exactly the k-slots of the P^T operand.
// The running max is only moved when the tile max exceeds it by more than
// 2^8 (the result is exact either way; it only bounds p <= 256), which keeps
// the O rescale off the common path.
//
// E4M3 instance (head_dim 128): the scores come from 8-bit codes, the
// SageAttention-style quantized attention the paper's §3.4 cites. Queries
// carry one scale per (token, head), the smoothed keys one per (64-key tile,
// head); K Q^T runs as 8 MFMA 32x32x64 per tile on the codes (a K tile is
// 8 KB: 128-byte rows, staged and swizzled like a 64-wide bf16 tile) and
// the product of the two scales joins the softmax scale in the one FMA per
// score that forms the exponent, so the softmax costs what it costs on bf16.
// V, P and P V are unchanged; the LSE outputs get the smoothing shift
// scale * q . mu added back.

#include <type_traits>

#include "device_common.h"
#include "ispa_internal.h"

namespace ispa {
namespace {

constexpr int kThreads = 512;              // 8 waves: 4 S-waves + 4 O-waves
constexpr int kPairs = 4;                  // (S-wave, O-wave) pairs
constexpr int kPairQ = 64;                 // queries per pair: two 32-query blocks
constexpr int kQTile = kPairs * kPairQ;    // queries per workgroup
constexpr int kKTile = 64;
constexpr float kRescaleThreshold = 8.0f;  // log2 units

// K and V tiles are staged in LDS in their natural [key][d] layout, with
// direct-to-LDS global loads (each wave instruction writes 64 lanes x 16 bytes
// contiguously), swizzled by lds_swz so that both the 16-byte K fragment
// reads and the transposing V reads are free of bank conflicts.
template <int D>
__device__ __forceinline__ int swz(int r) { return lds_swz<D>(r); }

struct Seg {
  const uint16_t* k;     // bf16 keys, or the E4M3 codes viewed as 16-bit pairs
  const uint16_t* v;
  int64_t n;
  const float* ksc;      // E4M3: scales [tiles][n_heads]
};

typedef int v8i32 __attribute__((ext_vector_type(8)));
typedef int v4i32_t __attribute__((ext_vector_type(4)));

// E4M3 K operand of a 64-key tile with 128-byte rows (a tile of 64-wide
// 16-bit rows, swizzled by lds_swz<64>): key row r, k-step t (64 channels),
// lane half h: channels 64 t + 32 h .. + 31, the logical 16-byte chunks
// 4 t + 2 h and 4 t + 2 h + 1.
__device__ __forceinline__ v8i32 k8_frag(const uint16_t* ks, int r, int t, int h) {
  const int sw = lds_swz<64>(r);
  const uint16_t* row = ks + r * 64;
  const v4i32_t lo = *reinterpret_cast<const v4i32_t*>(row + 8 * ((4 * t + 2 * h) ^ sw));
  const v4i32_t hi = *reinterpret_cast<const v4i32_t*>(row + 8 * ((4 * t + 2 * h + 1) ^ sw));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 32x32x64 E4M3 MFMA (both operands E4M3, no block scales): lane l holds the
// 32 consecutive k of row (A) / column (B) l % 32 from k = 32 (l / 32); the
// result layout is that of mfma32x32x16.
__device__ __forceinline__ f32x16 mfma_e4m3(v8i32 a, v8i32 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Direct-to-LDS loads of one 64-key tile of K and V. Each lane's byte offset
// inside a full tile is fixed, so a full tile only moves a uniform base.
// In a tail tile, rows past `valid` re-load the last valid row (in bounds);
// their scores are masked to -inf, so they contribute nothing.
template <int D, int NW>
struct TileLoader {
  static constexpr int CPR = D / 8;            // 16-byte chunks per key row
  static constexpr int RPI = 64 / CPR;         // rows per wave instruction
  static constexpr int IPW = kKTile / RPI / NW; // instructions per wave per tensor
  uint32_t off[IPW];                           // bytes, full tile
  int w, head, lds_base;                       // lds_base in elements

  // tile row and global column (elements) of the lane's chunk in instruction i
  __device__ int row_of(int i, int lane) const { return (w * IPW + i) * RPI + lane / CPR; }
  __device__ int col_of(int i, int lane) const {
    return head * D + 8 * ((lane % CPR) ^ swz<D>(row_of(i, lane)));
  }

  // `w_` in [0, NW): this wave's share of the tile rows (wave-uniform)
  __device__ void init(int64_t rs, int head_, int w_, int lane) {
    w = w_;
    head = head_;
    lds_base = w * IPW * RPI * D;
#pragma unroll
    for (int i = 0; i < IPW; ++i)
      off[i] = static_cast<uint32_t>((row_of(i, lane) * rs + col_of(i, lane)) * 2);
  }

  // Loads this wave's rows of one tile of K (issue_k) or V (issue_v).
  __device__ void issue_k(const Seg& sg, int64_t row0, int valid, int64_t rs,
                          uint16_t* dst) const {
    issue(sg.k, row0, valid, rs, dst);
  }
  __device__ void issue_v(const Seg& sg, int64_t row0, int valid, int64_t rs,
                          uint16_t* dst) const {
    issue(sg.v, row0, valid, rs, dst);
  }
  __device__ void issue(const uint16_t* src, int64_t row0, int valid, int64_t rs,
                        uint16_t* dst) const {
    const auto res = raw_rsrc(src + row0 * rs);
    if (valid == kKTile) {
#pragma unroll
      for (int i = 0; i < IPW; ++i) lds_dma16(res, dst + lds_base + i * RPI * D, off[i]);
    } else {
      const int lane = __lane_id();
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int r = row_of(i, lane);
        const int rr = r < valid ? r : valid - 1;
        lds_dma16(res, dst + lds_base + i * RPI * D,
                  static_cast<uint32_t>((rr * rs + col_of(i, lane)) * 2));
      }
    }
  }
};

// Three-way max in one instruction (the compiler does not always fuse the two
// maxima of a reduction chain); the inputs are finite scores.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

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

// Inverse of store_o: the bf16 values of a row block, as fp32.
template <int D>
__device__ __forceinline__ void load_o(const uint16_t* in, f32x16* o, int64_t qi, int64_t rs,
                                       int head, int hf) {
  const uint16_t* row = in + qi * rs + head * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint2 val = *reinterpret_cast<const uint2*>(row + 32 * db + 8 * g + 4 * hf);
      o[db][4 * g + 0] = __uint_as_float(val.x << 16);
      o[db][4 * g + 1] = __uint_as_float(val.x & 0xFFFF0000u);
      o[db][4 * g + 2] = __uint_as_float(val.y << 16);
      o[db][4 * g + 3] = __uint_as_float(val.y & 0xFFFF0000u);
    }
  }
}

// Feature-major form of store_o: element (query qi, feature
// head * D + d) at out[(head * D + d) * ld + qi]. Consecutive lanes hold
// consecutive queries, so each store covers 64 contiguous bytes of two rows.
// Buffer accesses with 32-bit byte offsets (a [h][ld] buffer stays below
// 2^31 bytes): one offset register per access instead of a 64-bit address.
template <int D>
__device__ __forceinline__ void store_ot(uint16_t* out, const f32x16* o, int64_t qi, int64_t ld,
                                         int head, int hf) {
  const auto rs = raw_rsrc(out);
  const uint32_t step = static_cast<uint32_t>(ld) * 2u;
  const uint32_t base = static_cast<uint32_t>(head * D + 4 * hf) * step +
                        static_cast<uint32_t>(qi) * 2u;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        __builtin_amdgcn_raw_buffer_store_b16(
            f32_to_bf16_bits(o[db][4 * g + r]), rs,
            static_cast<int>(base + static_cast<uint32_t>(32 * db + 8 * g + r) * step), 0, 0);
    // one 32-row block at a time: the conversions and offsets of all four
    // would otherwise be formed up front, at the register peak of the kernel
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One workgroup's work item `work` (head x query tile) of one attention call.
template <int D, bool F8>
__device__ __forceinline__ void attn_block(const AttnParams& p, const int work) {
  static_assert(!F8 || D == 128, "the E4M3 instance is built for head_dim 128");
  constexpr int TBUF = kKTile * D;   // one V tile (elements)
  constexpr int KD = F8 ? D / 2 : D; // K tile row in 16-bit units
  constexpr int TBUFK = kKTile * KD; // one K tile
  constexpr int NB = D / 32;         // 32-wide d blocks of O^T
  constexpr int NT = F8 ? D / 64 : D / 16;  // k-steps of K Q^T
  using KF = std::conditional_t<F8, v8i32, bf16x8>;  // K operand of one MFMA
  constexpr int PSLOT = kPairs * 2 * 4 * 64;  // P^T operands of one tile (16-byte units)
  // K and V tiles, two buffers each, and the P^T hand-off, two slots: every
  // access names a fixed array, so the compiler can see that a load into one
  // buffer never aliases the reads of another and needs no early wait.
  __shared__ __attribute__((aligned(16))) uint16_t sk0[TBUFK];
  __shared__ __attribute__((aligned(16))) uint16_t sk1[TBUFK];
  __shared__ __attribute__((aligned(16))) uint16_t sv0[TBUF];
  __shared__ __attribute__((aligned(16))) uint16_t sv1[TBUF];
  __shared__ uint4 sp0[PSLOT];                 // [pair][qb][st][lane]
  __shared__ uint4 sp1[PSLOT];
  __shared__ float sal0[kPairs * 128];         // rescale factor per lane [pair][hf][qb*32+q]
  __shared__ float sal1[kPairs * 128];
  __shared__ float s_inv_loc[kPairs * 64];     // 1 / l of the local phase
  __shared__ float s_inv_fin[kPairs * 64];     // 1 / l of the history (or only) phase
  __shared__ float s_wh[kPairs * 64];          // merge weight w_H

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, l32 = lane % 32, hf = lane / 32;
  const int pair = wave % kPairs;
  const bool s_role = wave < kPairs;
  const int head = work / p.n_qtiles;
  const int qt = work % p.n_qtiles;
  const int64_t rs = static_cast<int64_t>(p.n_heads) * D;
  int qi[2];  // query rows of the two blocks (n_q < 2^31)
  bool qvalid[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    qi[qb] = qt * kQTile + pair * kPairQ + 32 * qb + l32;
    qvalid[qb] = qi[qb] < p.n_q;
  }

  const int nt0 = static_cast<int>((p.n[0] + kKTile - 1) / kKTile);
  const int nt1 = static_cast<int>((p.n[1] + kKTile - 1) / kKTile);
  const int nt2 = static_cast<int>((p.n[2] + kKTile - 1) / kKTile);
  const int nt3 = static_cast<int>((p.n[3] + kKTile - 1) / kKTile);
  const int n_local_tiles = nt0 + nt1;
  const bool split = p.mode == 0;
  const bool run_hist = !(split && !p.need_hist);
  const int T = n_local_tiles + (run_hist ? nt2 + nt3 : 0);
  const bool has_hist = p.n[2] + p.n[3] > 0;

  auto tile_of = [&](int idx, Seg& sg, int64_t& row0, int& valid) {
    const int h0 = n_local_tiles + nt2;  // first tile of the second history piece
    const int g = idx < nt0 ? 0 : (idx < n_local_tiles ? 1 : (idx < h0 ? 2 : 3));
    const int t = idx - (g == 0 ? 0 : (g == 1 ? nt0 : (g == 2 ? n_local_tiles : h0)));
    sg.k = p.k[g];
    sg.v = p.v[g];
    sg.n = p.n[g];
    if constexpr (F8) {
      sg.k = reinterpret_cast<const uint16_t*>(p.k8[g]);
      sg.ksc = p.ksc[g];
    }
    row0 = static_cast<int64_t>(t) * kKTile;
    const int64_t rem = sg.n - row0;
    valid = rem < kKTile ? static_cast<int>(rem) : kKTile;
  };

  TileLoader<D, kPairs> loader;  // V, and K of the bf16 instance
  loader.init(rs, head, __builtin_amdgcn_readfirstlane(pair), lane);
  TileLoader<KD, kPairs> loader8;  // K codes of the E4M3 instance (rows of D bytes)
  if constexpr (F8) loader8.init(rs / 2, head, __builtin_amdgcn_readfirstlane(pair), lane);
  auto issue_k = [&](const Seg& sg, int64_t row0, int valid, uint16_t* dst) {
    if constexpr (F8)
      loader8.issue_k(sg, row0, valid, rs / 2, dst);
    else
      loader.issue_k(sg, row0, valid, rs, dst);
  };
  const int prow = pair * 64;  // this pair's entries in the per-query arrays
  const int prow2 = pair * 128;  // and in the per-lane rescale factors

  if (s_role) {
    // ------------------------------------------------------------ S-wave
    // Scores, online softmax statistics and P of every tile; P^T goes to the
    // pair's O-wave through LDS together with the rescale factors. The S-wave
    // runs one tile ahead of its own softmax: while the vector ALU works on
    // the scores of tile j, the matrix cores compute those of tile j+1, one
    // MFMA between consecutive slices of the softmax.
    bf16x8 qf[2][F8 ? 1 : NT];
    v8i32 qf8[2][F8 ? NT : 1];
    // E4M3: scale_log2 x the query's scale (times a tile's key scale, the
    // multiplier of the raw code products), and the smoothing shift of the LSE
    float qsl[2] = {p.scale_log2, p.scale_log2}, lcorr[2] = {0.f, 0.f};
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if constexpr (F8) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
          qf8[qb][t] = qvalid[qb] ? *reinterpret_cast<const v8i32*>(
                                        p.q8 + static_cast<int64_t>(qi[qb]) * rs + head * D +
                                        64 * t + 32 * hf)
                                  : v8i32{};
        qsl[qb] = qvalid[qb] ? p.scale_log2 * p.qsc[static_cast<int64_t>(head) * p.n_q + qi[qb]]
                             : 0.f;
        if (p.qmu && qvalid[qb]) lcorr[qb] = p.qmu[static_cast<int64_t>(head) * p.n_q + qi[qb]];
      } else {
#pragma unroll
        for (int t = 0; t < NT; ++t)
          qf[qb][t] = qvalid[qb] ? *reinterpret_cast<const bf16x8*>(
                                       p.q + static_cast<int64_t>(qi[qb]) * rs + head * D +
                                       16 * t + 8 * hf)
                                 : bf16x8{};
      }
    }
    // LSE output (natural log) of a log2-unit value
    auto lse_out = [&](float v2, int qb) {
      if constexpr (F8)
        return v2 * kLn2 + lcorr[qb];
      else
        return v2 * kLn2;
    };
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
    float lse_loc2[2] = {-INFINITY, -INFINITY};
    {
      Seg sg;
      int valid;
      int64_t row0;
      tile_of(0, sg, row0, valid);
      issue_k(sg, row0, valid, sk0);
      if (T > 1) {
        tile_of(1, sg, row0, valid);
        issue_k(sg, row0, valid, sk1);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // S^T[key half][query block] of the even (sa) and odd (sb) tiles
    f32x16 sa[2][2], sb[2][2];
    if constexpr (F8) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const v8i32 a0 = k8_frag(sk0, l32, t, hf), a1 = k8_frag(sk0, 32 + l32, t, hf);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          sa[0][qb] = mfma_e4m3(a0, qf8[qb][t], t ? sa[0][qb] : f32x16{});
          sa[1][qb] = mfma_e4m3(a1, qf8[qb][t], t ? sa[1][qb] : f32x16{});
        }
      }
    } else {
      bf16x8 a0 = k_frag<D>(sk0, l32, hf), a1 = k_frag<D>(sk0, 32 + l32, hf);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        bf16x8 n0, n1;
        if (t + 1 < NT) {
          n0 = k_frag<D>(sk0, l32, 2 * (t + 1) + hf);
          n1 = k_frag<D>(sk0, 32 + l32, 2 * (t + 1) + hf);
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          sa[0][qb] = mfma32x32x16(a0, qf[qb][t], t ? sa[0][qb] : f32x16{});
          sa[1][qb] = mfma32x32x16(a1, qf[qb][t], t ? sa[1][qb] : f32x16{});
        }
        a0 = n0;
        a1 = n1;
      }
    }
    __syncthreads();  // every wave is done with K of tile 0 before tile 2 replaces it

    // Softmax of one tile (scores sc) and, when QK, K Q^T of the next tile
    // (into sn, from K in ks). Slot u holds a slice of the softmax followed
    // by MFMA u; the scheduling barriers keep that order, so the vector work
    // runs while the matrix cores are busy.
    //   row max      (8 parts: query block x 4 scores of each key half)
    //   decision     (exchange between the lane halves, lazy rescale)
    //   exponentials (16 items: query block x key step x half)
    // A tail tile's rows past `valid` re-load the last valid key: their
    // scores duplicate real ones (the row maxima need no mask) and only
    // their exponentials are dropped, in a separate instance of this code.
    auto body = [&](auto tail_c, auto qk_c, f32x16(&sc)[2][2], f32x16(&sn)[2][2],
                    const uint16_t* __restrict__ ks, uint4* __restrict__ sp,
                    float* __restrict__ sal, int valid, const float(&cq)[2])
        __attribute__((always_inline)) {
      constexpr bool TAIL = decltype(tail_c)::value;
      constexpr bool QK = decltype(qk_c)::value;
      constexpr int NMF = 4 * NT;           // MFMAs of one tile's K Q^T
      constexpr int NMAX = NT >= 8 ? 4 : 2;  // slots of the row max
      constexpr int DEC = NMAX;             // slot of the rescale decision
      constexpr int E0 = DEC + 1;           // first slot of the exponentials
      float mx[2], lsum[2][4];
      bf16x8 pv;
      // Everything lane-dependent is derived from an opaque copy of the lane
      // index, so it is recomputed every tile instead of being hoisted out of
      // the tile loop and kept live (registers are the binding limit here).
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int r32 = ln & 31, h2 = ln >> 5;
      // K fragment of k-step t: row r32 (and r32 + 32), logical chunk 2t + h2,
      // stored at chunk (2t + h2) ^ swz = 2 (t ^ (swz >> 1)) + (h2 ^ (swz & 1))
      const int kf = r32 * D + 8 * (h2 ^ (swz<D>(r32) & 1));
      const int kx = 16 * (swz<D>(r32) >> 1);
      auto kfrag = [&](int t, int half) {
        if constexpr (F8)
          return k8_frag(ks, r32 + 32 * half, t, h2);
        else
          return *reinterpret_cast<const bf16x8*>(ks + kf + 32 * D * half + (kx ^ (16 * t)));
      };
      // operands of the two key halves, each read at the top of the slot two
      // slots before its first MFMA (the register being reloaded was last
      // read by the previous slot's MFMA)
      KF f0, f1;
      if constexpr (QK) {
        f0 = kfrag(0, 0);
        f1 = kfrag(0, 1);
      }
#pragma unroll
      for (int u = 0; u < NMF; ++u) {
        if constexpr (QK) {
          const int t = u / 4;
          if (u % 4 == 0 && u > 0) f1 = kfrag(t, 1);
          if (u % 4 == 2 && t + 1 < NT) f0 = kfrag(t + 1, 0);
        }
        // row max: one chain per query block (dependent max3 issue at full
        // rate), 8 parts of 4 scores of each key half
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          if (w * NMAX / 8 != u) continue;
          const int qb = w / 4, part = w % 4;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float a = sc[0][qb][4 * part + k], b = sc[1][qb][4 * part + k];
            if (part == 0 && k == 0)
              mx[qb] = fmaxf(a, b);
            else
              mx[qb] = max3(mx[qb], a, b);
          }
          // keep the slice in its slot (pure arithmetic is otherwise free to
          // move to its first use, which would leave the slots unbalanced and
          // keep every input live longer)
          asm volatile("" : "+v"(mx[qb]));
        }
        if (u == DEC) {
          // running max: moved only when the tile max exceeds it by more than
          // the threshold; the O-wave applies the same factor to its sums
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx[qb]),
                                                             __float_as_uint(mx[qb]), false, false);
            const float mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * cq[qb];
            const bool need = mt > m_run[qb] + kRescaleThreshold;
            const float alpha = need ? __builtin_amdgcn_exp2f(m_run[qb] - mt) : 1.f;
            m_run[qb] = need ? mt : m_run[qb];
            l_run[qb] *= alpha;
            sal[prow2 + 64 * h2 + 32 * qb + r32] = alpha;
          }
        }
        // P = 2^(s * scale_log2 - m): row sums in fp32 (the LSE needs them),
        // P^T to LDS rounded to bf16, lane-major in the MFMA operand layout
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          if (E0 + k * (NMF - E0) / 16 != u) continue;
          const int qb = k / 8, st = (k / 2) % 4, h = k % 2;
#pragma unroll
          for (int i = 4 * h; i < 4 * h + 4; ++i) {
            float e = __builtin_amdgcn_exp2f(
                fmaf(sc[st / 2][qb][8 * (st % 2) + i], cq[qb], -m_run[qb]));
            if constexpr (TAIL) {
              const int key = 32 * (st / 2) + 8 * ((8 * (st % 2) + i) / 4) + 4 * h2 + (i % 4);
              if (key >= valid) e = 0.f;
            }
            lsum[qb][st] = (h == 0 && i == 0) ? e : lsum[qb][st] + e;
            pv[i] = static_cast<__bf16>(e);
          }
          asm volatile("" : "+v"(lsum[qb][st]));
          if (h == 1) {
            sp[((pair * 2 + qb) * 4 + st) * 64 + ln] = __builtin_bit_cast(uint4, pv);
            l_run[qb] += lsum[qb][st];
          }
        }
        if constexpr (QK) {
          const int t = u / 4, kh = (u / 2) % 2, qb = u % 2;
          if constexpr (F8)
            sn[kh][qb] = mfma_e4m3(kh ? f1 : f0, qf8[qb][t], t ? sn[kh][qb] : f32x16{});
          else
            sn[kh][qb] = mfma32x32x16(kh ? f1 : f0, qf[qb][t], t ? sn[kh][qb] : f32x16{});
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (!QK) {
        // no next tile: its scores are never read, which the compiler cannot
        // see; redefining them keeps them from being live across the tile loop
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) asm volatile("" : "=v"(sn[kh][qb]));
      }
    };

    auto s_step = [&](auto buf_c, int it) __attribute__((always_inline)) {
      constexpr int BUF = decltype(buf_c)::value;
      const uint16_t* __restrict__ ks = BUF ? sk0 : sk1;  // K of tile it+1
      uint4* __restrict__ sp = BUF ? sp1 : sp0;
      float* __restrict__ sal = BUF ? sal1 : sal0;
      if (it < T) {
        Seg sg;
        int valid;
        int64_t row0;
        tile_of(it, sg, row0, valid);
        float cq[2] = {p.scale_log2, p.scale_log2};
        if constexpr (F8) {
          const float sk = sg.ksc[(row0 / kKTile) * p.n_heads + head];
          cq[0] = qsl[0] * sk;
          cq[1] = qsl[1] * sk;
        }
        auto run = [&](auto tail_c, auto qk_c) __attribute__((always_inline)) {
          if constexpr (BUF == 0)
            body(tail_c, qk_c, sa, sb, ks, sp, sal, valid, cq);
          else
            body(tail_c, qk_c, sb, sa, ks, sp, sal, valid, cq);
        };
        if (it + 1 < T) {
          if (valid == kKTile)
            run(std::false_type{}, std::true_type{});
          else
            run(std::true_type{}, std::true_type{});
        } else {
          if (valid == kKTile)
            run(std::false_type{}, std::false_type{});
          else
            run(std::true_type{}, std::false_type{});
        }

        if (split && it == n_local_tiles - 1) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32);
            lse_loc2[qb] = m_run[qb] + __builtin_amdgcn_logf(lt);
            if (hf == 0) s_inv_loc[prow + 32 * qb + l32] = 1.f / lt;
            if (qvalid[qb] && p.lse_local && hf == 0)
              p.lse_local[head * p.n_q + qi[qb]] = lse_out(lse_loc2[qb], qb);
            m_run[qb] = -INFINITY;
            l_run[qb] = 0.f;
          }
        }
      } else {
        // after the last tile: final statistics for the O-wave's epilogue
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32);
          float inv = 0.f, lse2 = -INFINITY, w_h = 0.f, lse_f2;
          if (!split) {
            inv = 1.f / lt;
            lse_f2 = m_run[qb] + __builtin_amdgcn_logf(lt);
          } else {
            if (has_hist) {
              inv = 1.f / lt;
              lse2 = m_run[qb] + __builtin_amdgcn_logf(lt);
            }
            lse_f2 = lse_loc2[qb];
            if (has_hist) {
              const float mm = fmaxf(lse_loc2[qb], lse2);
              lse_f2 = mm + __builtin_amdgcn_logf(__builtin_amdgcn_exp2f(lse_loc2[qb] - mm) +
                                                  __builtin_amdgcn_exp2f(lse2 - mm));
              w_h = __builtin_amdgcn_exp2f(lse2 - lse_f2);
            }
          }
          if (hf == 0) {
            s_inv_fin[prow + 32 * qb + l32] = inv;
            s_wh[prow + 32 * qb + l32] = w_h;
            if (qvalid[qb]) {
              if (split && p.need_hist && p.lse_hist)
                p.lse_hist[head * p.n_q + qi[qb]] = lse_out(lse2, qb);
              if ((!split || p.need_hist) && p.lse_full)
                p.lse_full[head * p.n_q + qi[qb]] = lse_out(lse_f2, qb);
            }
          }
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    };
    for (int it = 0; it <= T; it += 2) {
      s_step(std::integral_constant<int, 0>{}, it);
      if (it + 1 <= T) s_step(std::integral_constant<int, 1>{}, it + 1);
    }
    return;
  }

  // -------------------------------------------------------------- O-wave
  // O^T += V^T P^T one tile behind the S-wave, with its rescale factors.
  f32x16 oacc[2][NB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int b = 0; b < NB; ++b) oacc[qb][b] = f32x16{};
  // O_local is kept as its bf16 output values (the X the statistics see)
  // while the history phase runs, so D is formed against exactly that X: it
  // is parked in an output row this lane owns (O_local if requested, else
  // O_full, else D; each is written with its final value only after the
  // parked X has been read back). With none of them requested, no merge is
  // formed and X is not needed. The feature-major copies of X and D are
  // written in the epilogue from the parked X (the entry point that asks for
  // them always supplies O_full), which keeps their stores out of the tile
  // loop, where the O sums hold most of the registers.
  uint16_t* const park = p.o_local ? p.o_local : (p.o_full ? p.o_full : p.d_out);
  TrOff voff[NB];  // lane offsets of the V^T operand reads, per 32-wide d block
#pragma unroll
  for (int b = 0; b < NB; ++b) voff[b] = tr_offsets<D>(32 * b, lane);
  __syncthreads();  // K of tiles 0 and 1 staged (the S-waves' prologue)
  __syncthreads();  // K Q^T of tile 0 issued

  auto o_step = [&](auto buf_c, int it) {
    constexpr int BUF = decltype(buf_c)::value;
    const uint16_t* __restrict__ vs = BUF ? sv0 : sv1;   // V of tile it-1
    uint16_t* __restrict__ nvs = BUF ? sv1 : sv0;        // V of tile it
    uint16_t* __restrict__ nks = BUF ? sk1 : sk0;        // K of tile it+2
    const uint4* __restrict__ sp = BUF ? sp0 : sp1;      // P of tile it-1
    const float* __restrict__ sal = BUF ? sal0 : sal1;
    // the next tiles' loads go out after this step's P V: issued before it,
    // their LDS writes compete with the V and P operand reads of the MFMAs
    // for the LDS queues and stall them
    auto issue_loads = [&]() __attribute__((always_inline)) {
      if (it < T) {
        Seg sg;
        int valid;
        int64_t row0;
        tile_of(it, sg, row0, valid);
        loader.issue_v(sg, row0, valid, rs, nvs);
        if (it + 2 < T) {
          tile_of(it + 2, sg, row0, valid);
          issue_k(sg, row0, valid, nks);
        }
      }
    };
    if (it >= 1) {
      const int jb = it - 1;
      const float al0 = sal[prow2 + 64 * hf + l32], al1 = sal[prow2 + 64 * hf + 32 + l32];
      if (__any(al0 != 1.f || al1 != 1.f)) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          oacc[0][b] *= al0;
          oacc[1][b] *= al1;
        }
      }
      // V^T operands PD MFMA pairs ahead of their use (the LDS latency is
      // several MFMA pairs long), P^T operands one key step ahead
      constexpr int NU = 4 * NB;  // u = key step * NB + d block
      constexpr int PD = 3;
      auto pfrag = [&](int qb, int st) {
        return __builtin_bit_cast(bf16x8, sp[((pair * 2 + qb) * 4 + st) * 64 + lane]);
      };
      auto vfrag = [&](int u) { return tr_operand_at<D>(vs, 16 * (u / NB), voff[u % NB]); };
      bf16x8 vq[PD];
#pragma unroll
      for (int i = 0; i < PD; ++i) vq[i] = vfrag(i);
      bf16x8 p0 = pfrag(0, 0), p1 = pfrag(1, 0), q0, q1;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int st = u / NB, db = u % NB;
        const bf16x8 va = vq[u % PD];
        if (u + PD < NU) vq[u % PD] = vfrag(u + PD);
        if (db == 0 && st + 1 < 4) {
          q0 = pfrag(0, st + 1);
          q1 = pfrag(1, st + 1);
        }
        oacc[0][db] = mfma32x32x16(va, p0, oacc[0][db]);
        oacc[1][db] = mfma32x32x16(va, p1, oacc[1][db]);
        if (db == NB - 1) {
          p0 = q0;
          p1 = q1;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (split && jb == n_local_tiles - 1) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float inv = s_inv_loc[prow + 32 * qb + l32];
#pragma unroll
          for (int b = 0; b < NB; ++b) oacc[qb][b] *= inv;
          if (qvalid[qb] && park) store_o<D>(park, oacc[qb], qi[qb], rs, head, hf);
#pragma unroll
          for (int b = 0; b < NB; ++b) oacc[qb][b] = f32x16{};
        }
      }
    }
    issue_loads();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  for (int it = 0; it <= T; it += 2) {
    o_step(std::integral_constant<int, 0>{}, it);
    if (it + 1 <= T) o_step(std::integral_constant<int, 1>{}, it + 1);
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (!qvalid[qb]) continue;
    const float inv = s_inv_fin[prow + 32 * qb + l32];
    if (!split) {
#pragma unroll
      for (int b = 0; b < NB; ++b) oacc[qb][b] *= inv;
      if (p.o_full) store_o<D>(p.o_full, oacc[qb], qi[qb], rs, head, hf);
      continue;
    }
    if (!p.need_hist) continue;
    // history result (O_H = 0 for an empty history), then the LSE merge:
    // D = w_H (O_H - O_L), O_F = O_L + D
#pragma unroll
    for (int b = 0; b < NB; ++b) oacc[qb][b] *= inv;
    if (p.o_hist) store_o<D>(p.o_hist, oacc[qb], qi[qb], rs, head, hf);
    if (!park) continue;
    const float w_h = s_wh[prow + 32 * qb + l32];
    f32x16 xl[NB];
    load_o<D>(park, xl, qi[qb], rs, head, hf);
    if (p.xt) store_ot<D>(p.xt, xl, qi[qb], p.ldt, head, hf);
#pragma unroll
    for (int b = 0; b < NB; ++b) oacc[qb][b] = (oacc[qb][b] - xl[b]) * w_h;
    if (p.d_out) store_o<D>(p.d_out, oacc[qb], qi[qb], rs, head, hf);
    if (p.dt) store_ot<D>(p.dt, oacc[qb], qi[qb], p.ldt, head, hf);
    if (p.o_full) {
#pragma unroll
      for (int b = 0; b < NB; ++b) oacc[qb][b] += xl[b];
      store_o<D>(p.o_full, oacc[qb], qi[qb], rs, head, hf);
    }
  }
}

template <int D, bool F8>
__global__ __launch_bounds__(kThreads, 1) void attn_decomp_kernel(const AttnParams p) {
  attn_block<D, F8>(p, xcd_remap(blockIdx.x, gridDim.x));
}

// Several attention calls (instances, same heads) in one launch. The
// logical work order is head-major: for each head, the query tiles of call
// 0, then of call 1, ... (start[g] = query tiles of the calls before g).
// With the XCD remap each XCD takes a contiguous run of that order, so a
// head's query tiles of one call still share an XCD's L2, and every XCD
// gets a mix of all calls (calls with long histories are not piled onto a
// few XCDs).
template <int D, bool F8>
__global__ __launch_bounds__(kThreads, 1) void attn_grouped_kernel(const AttnGroup grp) {
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int per_head = grp.start[grp.n];
  const int head = t / per_head, r = t % per_head;
  int g = 0;
#pragma unroll 1
  while (g + 1 < grp.n && r >= grp.start[g + 1]) ++g;
  attn_block<D, F8>(grp.p[g], head * grp.p[g].n_qtiles + (r - grp.start[g]));
}

}  // namespace

hipError_t launch_attn_grouped(AttnGroup grp, int head_dim, hipStream_t stream) {
  if (grp.n < 1 || grp.n > kMaxGroup) return hipErrorInvalidValue;
  const bool f8 = grp.p[0].q8 != nullptr;
  const int n_heads = grp.p[0].n_heads;
  int64_t per_head = 0;
  for (int g = 0; g < grp.n; ++g) {
    AttnParams& p = grp.p[g];
    if ((p.q8 != nullptr) != f8 || p.n_heads != n_heads) return hipErrorInvalidValue;
    p.n_qtiles = static_cast<int>((p.n_q + kQTile - 1) / kQTile);
    grp.start[g] = static_cast<int>(per_head);
    per_head += p.n_qtiles;
  }
  grp.start[grp.n] = static_cast<int>(per_head);
  if (per_head * n_heads > INT32_MAX) return hipErrorInvalidValue;
  const int total = static_cast<int>(per_head * n_heads);
  if (total == 0) return hipSuccess;
  if (f8) {
    if (head_dim != 128) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_grouped_kernel<128, true>), dim3(total), dim3(kThreads), 0, stream,
                       grp);
  } else if (head_dim == 128) {
    hipLaunchKernelGGL((attn_grouped_kernel<128, false>), dim3(total), dim3(kThreads), 0, stream,
                       grp);
  } else {
    hipLaunchKernelGGL((attn_grouped_kernel<64, false>), dim3(total), dim3(kThreads), 0, stream,
                       grp);
  }
  return hipGetLastError();
}

hipError_t launch_attn_decomp(AttnParams p, int head_dim, hipStream_t stream) {
  p.n_qtiles = static_cast<int>((p.n_q + kQTile - 1) / kQTile);
  const int blocks = p.n_qtiles * p.n_heads;
  if (blocks == 0) return hipSuccess;
  if (p.q8) {
    if (head_dim != 128) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_decomp_kernel<128, true>), dim3(blocks), dim3(kThreads), 0, stream,
                       p);
  } else if (head_dim == 128) {
    hipLaunchKernelGGL((attn_decomp_kernel<128, false>), dim3(blocks), dim3(kThreads), 0, stream,
                       p);
  } else {
    hipLaunchKernelGGL((attn_decomp_kernel<64, false>), dim3(blocks), dim3(kThreads), 0, stream,
                       p);
  }
  return hipGetLastError();
}

int attn_q_tile_min() { return kQTile; }

}  // namespace ispa
