// 256 x 256-tile NT GEMM on bf16 matrix cores, fp32 accumulate:
//   out[m][n] = sum_k A[m][k] B[n][k]        (both operands k-contiguous)
// for the L-layer output projection Y = X W^T (ISPA paper §3.1 item 3), the
// warmup statistics G, C, E from feature-major activations X^T, D^T (§3.1
// item 2: the contraction runs over the tokens) and the fp32 x bf16
// products of the closed-form absorb (§3.2).
//
// Workgroup tile 256 x 256, 8 waves as 2 (m) x 4 (n) of 128 x 64 (4 x 2
// blocks of 32x32x16 MFMAs, 128 accumulators a lane; two waves a SIMD). Per
// 16-k step a wave reads 4 A and 2 B fragments (16 bytes a lane) for 8
// MFMAs: 0.75 KB of LDS reads per MFMA, against 1 KB for 64 x 64 wave
// tiles, and the tile's operand intensity (2 * 256 * 256 / (512 * 2 B) =
// 128 FLOP/B) halves the L2 -> CU stream of a 256 x 128 tile at the same
// rate.
//
// k-stages of 64 (128-byte LDS rows: each row of a stage is one whole L2
// line, so a stage takes half the cache requests of two 64-byte stages) go
// through two 64 KB LDS slots filled by direct-to-LDS buffer loads
// (lds_dma_asm.h) one stage ahead: each wave waits for its own loads of the
// stage it is about to read (vmcnt), one plain barrier per stage publishes
// them and frees the other slot, whose refill is spread between the first
// MFMAs. A row's 16-byte chunk c is stored at chunk position c ^ ((row >> 1)
// & 7), so the 16 rows of one quarter-wave's fragment reads cover all 64
// banks once. Rows past the matrix re-load its last row (their results are
// never stored). A contraction length that is not a multiple of 64 ends in a
// stage whose chunks past the end re-load the last valid chunk and whose
// fragment elements past the end are zeroed in registers. (The tile function
// also takes 32-k stages in a 4-slot ring filled three stages ahead.)

#include "device_common.h"
#include "ispa_internal.h"
#include "lds_dma_asm.h"

namespace ispa {
namespace {

constexpr int kBM = 256, kBN = 256;
// k per ring stage: 64 (128-byte rows, whole L2 lines, two 64 KB slots)
// measured 1.03-1.3x the rate of 32 (64-byte rows, four 32 KB slots) on the
// projection, the Gram and the split products
constexpr int kStageK = 64;
constexpr int kThreads = 512;
constexpr int kGroupM = 4;   // row tiles per L2 group

// Zero the elements of a fragment (8 consecutive k from k0) at k >= k_end.
__device__ __forceinline__ bf16x8 mask_k(bf16x8 f, int k0, int k_end) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (k0 + e >= k_end) f[e] = static_cast<__bf16>(0.f);
  return f;
}

}  // namespace

// One product (or one batch entry of it). Element (r, k) of A lives at
// a[r * lda + k]; of B at b[r * ldb + k]. a2: a second plane of A whose
// contraction follows the first one's with the same B (an fp32 operand held
// as hi + lo bf16 planes).
struct G256Args {
  const uint16_t* a;
  const uint16_t* a2;
  const uint16_t* b;
  int64_t lda, ldb;
  int64_t m;        // rows of A
  int n;            // rows of B
  int k;            // contraction length
  // output: bf16 or fp32 [m][n] with row stride ldy; for the accumulating
  // form, dest += (or = with zero_first) and, for a symmetric product
  // (A == B), only elements with row >= column are formed and each is also
  // written to its mirror position.
  void* y;
  int64_t ldy;
  int sym;
  int zero_first;
};

namespace {

enum { kOutBf16 = 0, kOutF32 = 1, kAccF32 = 2 };

template <int OUT, int KB, int BM>
__device__ __forceinline__ void g256_tile(const G256Args& p, const int tm, const int tn) {
  static_assert(KB == 32 || KB == 64, "stages of 32 or 64 k");
  static_assert(BM == 256 || BM == 192, "row tiles of 256 or 192");
  constexpr int NS = KB == 32 ? 4 : 2;   // ring slots (128 KB of LDS either way at BM 256)
  constexpr int CPR = KB / 8;            // 16-byte chunks of an LDS row
  constexpr int RPI = 64 / CPR;          // rows one load instruction fills
  constexpr int RWA = BM / 8;            // A rows a wave loads per stage
  constexpr int LPWA = RWA / RPI;        // load instructions a wave issues for A
  constexpr int LPWB = 32 / RPI;         // ... for B
  constexpr int LS = LPWA + LPWB;        // ... per stage
  constexpr int KS = KB / 16;            // MFMA k-steps of a stage
  constexpr int MI = BM / 64;            // 32-row MFMA blocks of a wave (its rows: BM / 2)
  static_assert(RWA % RPI == 0, "whole load instructions per wave");
  __shared__ __attribute__((aligned(16))) uint16_t sa[NS][BM * KB];
  __shared__ __attribute__((aligned(16))) uint16_t sb[NS][kBN * KB];
  // chunk c of row r sits at position c ^ swz(r): the 16 rows of a
  // quarter-wave's fragment reads then cover the 64 banks once
  auto pos_of = [](int r, int c) {
    return KB == 32 ? c ^ ((r >> 2) & 3) : c ^ ((r >> 1) & 7);
  };

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, l32 = lane % 32, hf = lane / 32;
  const int wm = wave / 4, wn = wave % 4;
  const int64_t m0 = static_cast<int64_t>(tm) * BM;
  const int n0 = tn * kBN;

  const int nk = (p.k + KB - 1) / KB;
  const bool tail = (p.k % KB) != 0;
  const int nst = p.a2 ? 2 * nk : nk;
  const u32x4 ra1 = desc_of(p.a);
  const u32x4 ra2 = desc_of(p.a2 ? p.a2 : p.a);
  const u32x4 rb = desc_of(p.b);

  // wave w loads A rows [RWA w, RWA w + RWA) and B rows [32 w, 32 w + 32) of
  // a stage, LPWA and LPWB instructions; lane -> (row lane / CPR, position
  // lane % CPR)
  uint32_t va[LPWA], vb[LPWB];
  int lrowa[LPWA], lrowb[LPWB];
  const int pc = lane % CPR;
#pragma unroll
  for (int j = 0; j < LPWA; ++j) {
    const int row = wave * RWA + RPI * j + lane / CPR;
    lrowa[j] = row;
    int64_t gr = m0 + row;
    if (gr > p.m - 1) gr = p.m - 1;
    va[j] = static_cast<uint32_t>(gr * p.lda * 2 + 16 * pos_of(row, pc));
  }
#pragma unroll
  for (int j = 0; j < LPWB; ++j) {
    const int row = wave * 32 + RPI * j + lane / CPR;
    lrowb[j] = row;
    int gb = n0 + row;
    if (gb > p.n - 1) gb = p.n - 1;
    vb[j] = static_cast<uint32_t>(static_cast<int64_t>(gb) * p.ldb * 2 + 16 * pos_of(row, pc));
  }
  // the last stage of a ragged contraction: chunks that start past the end
  // re-load the last valid chunk (in bounds; masked after the read)
  const int k_last_chunk = ((p.k - 1) / 8) * 8;
  auto tail_off = [&](uint32_t v, int row, int kst) {
    const int c = pos_of(row, pc);
    int k0 = kst * KB + 8 * c;
    if (k0 > k_last_chunk) k0 = k_last_chunk;
    return v - 16 * c + 2 * k0;   // same row, chunk at k0 (stage offset not added)
  };
  // load j (0 .. LS - 1) of stage s into slot (da, db): j < LPWA A, else B
  auto dma = [&](int s, uint16_t* da, uint16_t* db, int j) __attribute__((always_inline)) {
    const int kst = s >= nk ? s - nk : s;
    const bool t = tail && kst == nk - 1;
    if (j < LPWA) {
      const int row0 = wave * RWA + RPI * j;
      const u32x4 r = s >= nk ? ra2 : ra1;
      dma16_asm(r, da + row0 * KB, t ? tail_off(va[j], lrowa[j], kst) : va[j],
                t ? 0 : kst * 2 * KB);
    } else {
      const int jj = j - LPWA;
      const int row0 = wave * 32 + RPI * jj;
      dma16_asm(rb, db + row0 * KB, t ? tail_off(vb[jj], lrowb[jj], kst) : vb[jj],
                t ? 0 : kst * 2 * KB);
    }
  };

  f32x16 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  int ar[MI], br[2], apos[MI][KS], bpos[2][KS];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    ar[i] = wm * (BM / 2) + i * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) apos[i][kk] = pos_of(ar[i], 2 * kk + hf);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    br[j] = wn * 64 + j * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) bpos[j][kk] = pos_of(br[j], 2 * kk + hf);
  }
  auto frag_at = [](const uint16_t* slot, int row, int pos) {
    return *reinterpret_cast<const bf16x8*>(slot + row * KB + 8 * pos);
  };

  for (int s = 0; s < NS - 1 && s < nst; ++s)
#pragma unroll
    for (int j = 0; j < LS; ++j) dma(s, sa[s], sb[s], j);

  auto stage = [&](int s, const uint16_t* __restrict__ ca, const uint16_t* __restrict__ cb,
                   uint16_t* __restrict__ na, uint16_t* __restrict__ nb)
      __attribute__((always_inline)) {
    // this wave's loads of stage s have landed; the stages issued after it
    // (up to NS - 2 of them, LS loads each) may stay in flight
    if constexpr (NS == 4) {
      if (s + 2 < nst)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else if (s + 1 < nst)
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    // a plain barrier: __syncthreads() would add a wait for every load in
    // flight, including the stages issued ahead
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int kst = s >= nk ? s - nk : s;
    const bool mask = tail && kst == nk - 1;
    const bool refill = s + NS - 1 < nst;
    // two k-steps at a time: their fragments, then their MFMAs, the refill of
    // the slot freed by the previous stage spread between the first ones
#pragma unroll
    for (int h2 = 0; h2 < KS / 2; ++h2) {
      bf16x8 av[2][MI], bv[2][2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int kk = 2 * h2 + q;
#pragma unroll
        for (int i = 0; i < MI; ++i) av[q][i] = frag_at(ca, ar[i], apos[i][kk]);
#pragma unroll
        for (int j = 0; j < 2; ++j) bv[q][j] = frag_at(cb, br[j], bpos[j][kk]);
        if (mask) {
          const int k0 = kst * KB + 16 * kk + 8 * hf;
#pragma unroll
          for (int i = 0; i < MI; ++i) av[q][i] = mask_k(av[q][i], k0, p.k);
#pragma unroll
          for (int j = 0; j < 2; ++j) bv[q][j] = mask_k(bv[q][j], k0, p.k);
        }
      }
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            acc[i][j] = mfma32x32x16(av[q][i], bv[q][j], acc[i][j]);
            const int u = (h2 * 2 + q) * (2 * MI) + i * 2 + j;
            if (u < LS && refill) dma(s + NS - 1, na, nb, u);
          }
    }
  };
  for (int s0 = 0; s0 < nst; s0 += NS) {
#pragma unroll
    for (int q = 0; q < NS; ++q)
      if (s0 + q < nst) stage(s0 + q, sa[q], sb[q], sa[(q + NS - 1) % NS], sb[(q + NS - 1) % NS]);
  }

  // epilogue: lane holds rows 8 (r / 4) + 4 hf + r % 4 of each 32-row block
  // and column l32 of each 32-column block
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + l32;
      if (n >= p.n) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t mb = m0 + wm * (BM / 2) + i * 32 + 8 * g + 4 * hf;
        if constexpr (OUT == kOutBf16) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (mb + r < p.m)
              static_cast<uint16_t*>(p.y)[(mb + r) * p.ldy + n] =
                  f32_to_bf16_bits(acc[i][j][4 * g + r]);
        } else if constexpr (OUT == kOutF32) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (mb + r < p.m) static_cast<float*>(p.y)[(mb + r) * p.ldy + n] = acc[i][j][4 * g + r];
        } else {
          float* d = static_cast<float*>(p.y);
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * g + r];
          // direct elements (row >= column when symmetric)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t m = mb + r;
            if (m >= p.m || (p.sym && m < n)) continue;
            float* c = d + m * p.ldy + n;
            *c = p.zero_first ? v[r] : *c + v[r];
          }
          // mirror elements (row > column): 4 consecutive columns of row n
          if (p.sym) {
            if (mb > n && mb + 3 < p.m) {
              float4* c = reinterpret_cast<float4*>(d + static_cast<int64_t>(n) * p.ldy + mb);
              float4 o = make_float4(v[0], v[1], v[2], v[3]);
              if (!p.zero_first) {
                const float4 old = *c;
                o.x += old.x; o.y += old.y; o.z += old.z; o.w += old.w;
              }
              *c = o;
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int64_t m = mb + r;
                if (m >= p.m || m <= n) continue;
                float* c = d + static_cast<int64_t>(n) * p.ldy + m;
                *c = p.zero_first ? v[r] : *c + v[r];
              }
            }
          }
        }
      }
    }
  }
}

// Row tile tm and column tile tn of logical tile t in grouped order:
// kGroupM row tiles share each column panel.
__device__ __forceinline__ void grouped_tile(int t, int tiles_m, int tiles_n, int* tm, int* tn) {
  const int per_group = kGroupM * tiles_n;
  const int g = t / per_group, first_m = g * kGroupM;
  const int gm = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
  *tm = first_m + (t % per_group) % gm;
  *tn = (t % per_group) / gm;
}

template <int OUT, int KB, int BM>
__global__ __launch_bounds__(kThreads, 1) void g256_kernel(const G256Args p, int64_t a_bs,
                                                           int64_t a2_bs, int64_t b_bs,
                                                           int64_t y_bs) {
  const int tiles_m = static_cast<int>((p.m + BM - 1) / BM);
  const int tiles_n = (p.n + kBN - 1) / kBN;
  int tm, tn;
  grouped_tile(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, &tm, &tn);
  const int64_t b = blockIdx.y;
  G256Args q = p;
  q.a = p.a + b * a_bs;
  q.a2 = p.a2 ? p.a2 + b * a2_bs : nullptr;
  q.b = p.b + b * b_bs;
  q.y = static_cast<char*>(p.y) + b * y_bs * (OUT == kOutBf16 ? 2 : 4);
  g256_tile<OUT, KB, BM>(q, tm, tn);
}

// Tile u of a lower triangle of nt x nt tiles in grouped order: groups of
// kGroupM tile rows, each swept column by column over the tiles on or below
// the diagonal, so that consecutive tiles share row panels as in
// grouped_tile (row-major order would give a window of consecutive tiles in
// the last rows one column panel per tile).
__device__ __forceinline__ void tri_grouped_tile(int u, int nt, int* tm, int* tn) {
  int r0 = 0, gm = 0;
  for (;; r0 += kGroupM) {
    gm = nt - r0 < kGroupM ? nt - r0 : kGroupM;
    const int cnt = gm * r0 + gm * (gm + 1) / 2;
    if (u < cnt) break;
    u -= cnt;
  }
  if (u < gm * r0) {   // columns left of the group's diagonal block: gm tiles each
    *tn = u / gm;
    *tm = r0 + u % gm;
    return;
  }
  u -= gm * r0;        // the diagonal block: column r0 + j holds gm - j tiles
  int j = 0;
  while (u >= gm - j) {
    u -= gm - j;
    ++j;
  }
  *tn = r0 + j;
  *tm = r0 + j + u;
}

// The warmup statistics of one batch entry (layer) per blockIdx.y from
// feature-major X^T, D^T [h][ld]: the G tiles (lower triangle of 256-tiles,
// mirrored), the C tiles (all) and the E tiles (lower triangle, mirrored),
// each in an order whose consecutive tiles share operand panels.
struct GramTArgs {
  const uint16_t* xt;
  const uint16_t* dt;
  int64_t ld;          // row stride of X^T, D^T (elements)
  int64_t in_bs;       // batch stride of X^T, D^T (elements)
  int64_t n_tok;
  int h;
  float* G;
  float* C;
  float* E;            // may be null
  int zero_first;
};

template <int KB>
__global__ __launch_bounds__(kThreads, 1) void gram_t_kernel(const GramTArgs p, int nt,
                                                             int n_tiles) {
  const int t = xcd_remap(blockIdx.x, n_tiles);
  const int64_t b = blockIdx.y;
  const int n_sym = nt * (nt + 1) / 2;
  const int64_t hh = static_cast<int64_t>(p.h) * p.h;
  // order: C tiles (grouped), then G, then E (lower triangles, grouped)
  int job, tm, tn;
  if (t < nt * nt) {
    job = 1;
    grouped_tile(t, nt, nt, &tm, &tn);
  } else {
    int u = t - nt * nt;
    job = u < n_sym ? 0 : 2;
    if (u >= n_sym) u -= n_sym;
    tri_grouped_tile(u, nt, &tm, &tn);
  }
  G256Args q{};
  const uint16_t* xb = p.xt + b * p.in_bs;
  const uint16_t* db = p.dt + b * p.in_bs;
  q.a = job == 2 ? db : xb;
  q.a2 = nullptr;
  q.b = job == 0 ? xb : db;
  q.lda = q.ldb = p.ld;
  q.m = p.h;
  q.n = p.h;
  q.k = static_cast<int>(p.n_tok);
  q.y = (job == 0 ? p.G : (job == 1 ? p.C : p.E)) + b * hh;
  q.ldy = p.h;
  q.sym = job != 1;
  q.zero_first = p.zero_first;
  g256_tile<kAccF32, KB, kBM>(q, tm, tn);
}

// Buffer-load offsets are 32 bit: rows of A run in blocks whose bytes stay
// below 2^31 (a launch each); B must fit below 2^31 bytes as a whole.
template <int OUT, int BM = kBM>
hipError_t launch_g256(G256Args a, int batch, int64_t a_bs, int64_t b_bs, int64_t y_bs,
                       hipStream_t stream) {
  const int64_t row_bytes = a.lda * 2;
  const int64_t max_rows = (static_cast<int64_t>(INT32_MAX) / row_bytes) / BM * BM;
  if (max_rows == 0 || static_cast<int64_t>(a.n) * a.ldb * 2 > INT32_MAX)
    return hipErrorInvalidValue;
  if (batch == 0 || a.m == 0 || a.n == 0) return hipSuccess;
  const int64_t ys = OUT == kOutBf16 ? 2 : 4;
  for (int64_t r0 = 0; r0 < a.m; r0 += max_rows) {
    G256Args blk = a;
    blk.m = a.m - r0 < max_rows ? a.m - r0 : max_rows;
    blk.a = a.a + r0 * a.lda;
    if (a.a2) blk.a2 = a.a2 + r0 * a.lda;
    blk.y = static_cast<char*>(a.y) + r0 * a.ldy * ys;
    const int64_t tiles = ((blk.m + BM - 1) / BM) * ((a.n + kBN - 1) / kBN);
    hipLaunchKernelGGL((g256_kernel<OUT, kStageK, BM>), dim3(static_cast<unsigned>(tiles), batch),
                       dim3(kThreads), 0, stream, blk, a_bs, a_bs, b_bs, y_bs);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_g256_bf16(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t n,
                            int h_in, int h_out, hipStream_t stream, int row_tile) {
  G256Args a{};
  a.a = x;
  a.b = w;
  a.lda = a.ldb = h_in;
  a.m = n;
  a.n = h_out;
  a.k = h_in;
  a.y = y;
  a.ldy = h_out;
  if (row_tile == 192) return launch_g256<kOutBf16, 192>(a, 1, 0, 0, 0, stream);
  return launch_g256<kOutBf16>(a, 1, 0, 0, 0, stream);
}

hipError_t launch_g256_split_f32(const uint16_t* hi, const uint16_t* lo, const uint16_t* w,
                                 float* y, int h, int batch, hipStream_t stream) {
  const int64_t hh = static_cast<int64_t>(h) * h;
  G256Args a{};
  a.a = hi;
  a.a2 = lo;
  a.b = w;
  a.lda = a.ldb = h;
  a.m = h;
  a.n = h;
  a.k = h;
  a.y = y;
  a.ldy = h;
  return launch_g256<kOutF32>(a, batch, hh, hh, hh, stream);
}

hipError_t launch_gram_t(const uint16_t* xt, const uint16_t* dt, int64_t n_tok, int64_t ld, int h,
                         int batch, float* G, float* C, float* E, int zero_first,
                         hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  if (static_cast<int64_t>(h) * ld * 2 > INT32_MAX || ld % 8 != 0 || n_tok > ld)
    return hipErrorInvalidValue;
  const int nt = (h + kBM - 1) / kBM;
  const int n_sym = nt * (nt + 1) / 2;
  const int n_tiles = nt * nt + n_sym + (E ? n_sym : 0);
  GramTArgs p{xt, dt, ld, static_cast<int64_t>(h) * ld, n_tok, h, G, C, E, zero_first};
  hipLaunchKernelGGL(gram_t_kernel<kStageK>, dim3(n_tiles, batch), dim3(kThreads), 0, stream, p,
                     nt, n_tiles);
  return hipGetLastError();
}

}  // namespace ispa
