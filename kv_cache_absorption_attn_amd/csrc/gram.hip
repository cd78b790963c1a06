// Warmup statistics and the L-layer projection on CDNA4 bf16 matrix cores.
//
// Gram accumulation (ISPA paper §3.1 item 2: the accumulated dual-stream
// activations are the basis of the weight adaption): for X = O_local and
// D = O_full - O_local of one warmup step, G += X^T X, C += X^T D, E += D^T D,
// in fp32. Without D (G-only mode) the same kernel forms X^T X alone; the
// layer score uses it for W_o^T W_o. Treating Y = [X | D] as one [n_tok, 2h] matrix, every needed block
// is a 128 x 128 tile (bi <= bj) of the symmetric Y^T Y: both-X tiles feed G,
// X-D tiles feed C, both-D tiles feed E. Off-diagonal tiles of G and E are
// also added, transposed, into the mirror tile so G and E stay exactly
// symmetric. The contraction runs over tokens, so both operands are staged
// token-contiguous (Y^T) in LDS; the summation order is fixed (no atomics).
//
// Projection (ISPA paper §3.1 item 3: L-layers run with W_new = W + dW):
// Y = X W^T for nn.Linear-layout W, bf16 in, fp32 accumulate, bf16 out.

#include "device_common.h"
#include "ispa_internal.h"

namespace ispa {
namespace {

constexpr int kThreads = 256;
constexpr int kT = 128;          // output tile edge
constexpr int kTok = 64;         // tokens per LDS stage
constexpr int kBuf = kTok * kT;  // elements of one operand stage (16 KB)
constexpr int kGroup = 8;        // tile-order group edge (L2 panel sharing)

// Direct-to-LDS loads of one stage of a 128-feature block of Y (token-major
// rows of 256 bytes, swizzled as lds_swz<128>). Each wave instruction writes
// 4 rows. Features past the block's end are clamped to a valid column (they
// only feed outputs that are never stored); tokens past n_tok are clamped
// here and zeroed in LDS afterwards.
struct GramLoader {
  int row[4];
  uint32_t off[4];  // byte offset of the lane's 16-byte chunk from the stage's first row
  int col[4];       // element offset of that chunk within the block
  __device__ void init(int wave, int lane, int fvalid, int h) {
    const int p = lane % 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      row[i] = (wave * 4 + i) * 4 + lane / 16;
      int c = p ^ lds_swz<kT>(row[i]);
      if (8 * c >= fvalid) c = fvalid / 8 - 1;
      col[i] = 8 * c;
      off[i] = static_cast<uint32_t>((row[i] * h + col[i]) * 2);
    }
  }
  // A full stage: a uniform base plus the fixed lane offsets.
  __device__ void issue(const uint16_t* src, int h, int64_t t0, uint16_t* dst, int wave) const {
    const auto res = raw_rsrc(src + t0 * h);
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_dma16(res, dst + (wave * 4 + i) * 4 * kT, off[i]);
  }
  // The last (partial) stage: token rows past n_tok re-load the last token.
  __device__ void issue_tail(const uint16_t* src, int h, int64_t t0, int64_t n_tok, uint16_t* dst,
                             int wave) const {
    const auto res = raw_rsrc(src + t0 * h);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t t = t0 + row[i];
      if (t >= n_tok) t = n_tok - 1;
      lds_dma16(res, dst + (wave * 4 + i) * 4 * kT,
                static_cast<uint32_t>(((t - t0) * h + col[i]) * 2));
    }
  }
};

// Zero rows [valid, kTok) of a stage buffer (tail stage only).
__device__ __forceinline__ void zero_rows(uint16_t* buf, int valid, int tid) {
  for (int e = valid * (kT / 8) + tid; e < kTok * (kT / 8); e += kThreads)
    *reinterpret_cast<uint4*>(buf + 8 * e) = make_uint4(0, 0, 0, 0);
}

__global__ __launch_bounds__(kThreads, 2) void gram_kernel(const GramParams p, int nbp,
                                                            int n_tiles) {
  // 4 operand stages (A0 A1 B0 B1, 16 KB each); after the contraction the
  // same 64 KB (+ padding) holds the fp32 output tile for the epilogue.
  __shared__ __attribute__((aligned(16))) uint16_t stage_buf[4 * kBuf + 2 * 4 * kT];
  uint16_t* sa0 = stage_buf;
  uint16_t* sa1 = stage_buf + kBuf;
  uint16_t* sb0 = stage_buf + 2 * kBuf;
  uint16_t* sb1 = stage_buf + 3 * kBuf;

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, l32 = lane % 32, hf = lane / 32;
  const int wm = wave / 2, wn = wave % 2;
  const int b = blockIdx.y;

  // tile id -> (bi, bj), bi <= bj, over the 2*nbp block rows of Y^T Y. Tiles
  // are ordered in groups of kGroup x kGroup (upper-triangle groups, row-major)
  // and each XCD takes a contiguous range of ids, so the ~64 tiles resident on
  // one XCD cover about kGroup row panels and kGroup column panels of Y: the
  // panels are fetched once into that XCD's L2 and shared, instead of every
  // tile streaming its own column panel.
  int idx = xcd_remap(blockIdx.x, n_tiles);
  const int nb2 = p.d ? 2 * nbp : nbp;  // without D only the X X^T blocks (G)
  const int ng = (nb2 + kGroup - 1) / kGroup;
  int bi = 0, bj = 0;
  for (int gi = 0; gi < ng; ++gi) {
    const int ri = min(kGroup, nb2 - gi * kGroup);
    int gj = gi;
    for (; gj < ng; ++gj) {
      const int rj = min(kGroup, nb2 - gj * kGroup);
      const int size = gj == gi ? ri * (ri + 1) / 2 : ri * rj;
      if (idx < size) break;
      idx -= size;
    }
    if (gj == ng) continue;
    if (gj == gi) {  // upper triangle of a diagonal group, row by row
      int i = 0;
      while (idx >= ri - i) {
        idx -= ri - i;
        ++i;
      }
      bi = gi * kGroup + i;
      bj = bi + idx;
    } else {
      const int rj = min(kGroup, nb2 - gj * kGroup);
      bi = gi * kGroup + idx / rj;
      bj = gj * kGroup + idx % rj;
    }
    break;
  }

  const int h = p.h;
  const int64_t hh = static_cast<int64_t>(h) * h;
  const uint16_t* xb = p.x + b * p.n_tok * h;
  const uint16_t* db = p.d ? p.d + b * p.n_tok * h : xb;
  const bool i_is_d = bi >= nbp, j_is_d = bj >= nbp;
  const int fi0 = (i_is_d ? bi - nbp : bi) * kT;
  const int fj0 = (j_is_d ? bj - nbp : bj) * kT;
  const uint16_t* srci = (i_is_d ? db : xb) + fi0;
  const uint16_t* srcj = (j_is_d ? db : xb) + fj0;
  const int fvi = min(kT, h - fi0), fvj = min(kT, h - fj0);
  float* dest;
  if (!i_is_d && !j_is_d) dest = p.G + b * hh;
  else if (!i_is_d) dest = p.C + b * hh;
  else dest = p.E ? p.E + b * hh : nullptr;
  if (dest == nullptr) return;

  GramLoader li, lj;
  li.init(wave, lane, fvi, h);
  lj.init(wave, lane, fvj, h);
  TrOff oa[2], ob[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    oa[i] = tr_offsets<kT>(wm * 64 + i * 32, lane);
    ob[i] = tr_offsets<kT>(wn * 64 + i * 32, lane);
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nst = static_cast<int>((p.n_tok + kTok - 1) / kTok);
  const int tail = static_cast<int>(p.n_tok - static_cast<int64_t>(nst - 1) * kTok);
  auto issue_stage = [&](int s, uint16_t* da, uint16_t* db_) {
    const int64_t t0 = static_cast<int64_t>(s) * kTok;
    if (t0 + kTok <= p.n_tok) {
      li.issue(srci, h, t0, da, wave);
      lj.issue(srcj, h, t0, db_, wave);
    } else {
      li.issue_tail(srci, h, t0, p.n_tok, da, wave);
      lj.issue_tail(srcj, h, t0, p.n_tok, db_, wave);
    }
  };
  if (nst > 0) {
    issue_stage(0, sa0, sb0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (nst == 1 && tail < kTok) {
      zero_rows(sa0, tail, tid);
      zero_rows(sb0, tail, tid);
      __syncthreads();
    }
  }

  // One stage: contract 64 tokens of the buffers (ra, rb) while the next
  // stage lands in (na, nb). Restrict pointers: the buffer being filled never
  // aliases the ones being read, so the reads need not wait for the loads.
  auto stage = [&](int s, const uint16_t* __restrict__ ra, const uint16_t* __restrict__ rb,
                   uint16_t* __restrict__ na, uint16_t* __restrict__ nb) {
    const bool has_next = s + 1 < nst;
    if (has_next) issue_stage(s + 1, na, nb);
    // operands of the next 16 tokens are read while this step's MFMAs run
    bf16x8 a[2], bv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = tr_operand_at<kT>(ra, 0, oa[i]);
#pragma unroll
    for (int j = 0; j < 2; ++j) bv[j] = tr_operand_at<kT>(rb, 0, ob[j]);
#pragma unroll
    for (int st = 0; st < kTok / 16; ++st) {
      bf16x8 na[2], nbv[2];
      if (st + 1 < kTok / 16) {
#pragma unroll
        for (int i = 0; i < 2; ++i) na[i] = tr_operand_at<kT>(ra, 16 * (st + 1), oa[i]);
#pragma unroll
        for (int j = 0; j < 2; ++j) nbv[j] = tr_operand_at<kT>(rb, 16 * (st + 1), ob[j]);
      }
      // keeps the reads above the MFMAs (the scheduler would otherwise sink
      // them next to their use)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(a[i], bv[j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = na[i];
        bv[i] = nbv[i];
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (has_next && s + 2 == nst && tail < kTok) {
      zero_rows(na, tail, tid);
      zero_rows(nb, tail, tid);
      __syncthreads();
    }
  };
  for (int s = 0; s < nst; ++s) {
    const bool odd = s & 1;
    stage(s, odd ? sa1 : sa0, odd ? sb1 : sb0, odd ? sa0 : sa1, odd ? sb0 : sb1);
  }

  // Epilogue through LDS: the finished 128 x 128 fp32 tile is staged in the
  // (now idle) operand buffers, then added to dest(fi0 + m, fj0 + n) with
  // row-contiguous float4 accesses, and - for off-diagonal G / E tiles - to
  // the mirror tile dest(fj0 + n, fi0 + m), read back transposed.
  constexpr int kLd = kT + 4;   // fp32 row stride of the staged tile
  float* st = reinterpret_cast<float*>(stage_buf);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = wn * 64 + j * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm * 64 + i * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
        st[m * kLd + n] = acc[i][j][r];
      }
    }
  __syncthreads();
  const bool mirror = (i_is_d == j_is_d) && bi != bj;
  // direct tile: thread -> (row m, 4 columns); 32 float4 per row
  for (int e = tid; e < kT * (kT / 4); e += kThreads) {
    const int m = e / (kT / 4), n4 = (e % (kT / 4)) * 4;
    if (m >= fvi || n4 >= fvj) continue;
    const float* sv = st + m * kLd + n4;
    float4 v = make_float4(sv[0], sv[1], sv[2], sv[3]);
    float4* c = reinterpret_cast<float4*>(dest + static_cast<int64_t>(fi0 + m) * h + fj0 + n4);
    if (!p.zero_first) {
      const float4 o = *c;
      v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
    }
    *c = v;
  }
  if (mirror) {
    // mirror tile: thread -> (row n, 4 columns m)
    for (int e = tid; e < kT * (kT / 4); e += kThreads) {
      const int n = e / (kT / 4), m4 = (e % (kT / 4)) * 4;
      if (n >= fvj || m4 >= fvi) continue;
      float4 v = make_float4(st[m4 * kLd + n], st[(m4 + 1) * kLd + n], st[(m4 + 2) * kLd + n],
                             st[(m4 + 3) * kLd + n]);
      float4* c = reinterpret_cast<float4*>(dest + static_cast<int64_t>(fj0 + n) * h + fi0 + m4);
      if (!p.zero_first) {
        const float4 o = *c;
        v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
      }
      *c = v;
    }
  }
}

// ---------------------------------------------------------------- projection
constexpr int kPK = 32;           // k per stage (projection)
constexpr int kPStr = kPK + 8;    // LDS row stride (bf16)

// NT GEMM on bf16 matrix cores, fp32 accumulate: Y[m][o] = sum_k A[m][k] W[o][k]
// (both operands k-contiguous), batched over blockIdx.y. F32OUT = false: Y is
// bf16 (the projection). F32OUT = true: Y is fp32 and, when a2 is given, the
// A operand is a + a2 (two bf16 planes of an fp32 matrix: the contraction
// runs over both with the same W), i.e. an fp32 x bf16 product.
template <bool F32OUT>
__global__ __launch_bounds__(kThreads, 2) void nt_gemm_kernel(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ a2, int64_t a_bs,
    const uint16_t* __restrict__ w, int64_t w_bs, void* __restrict__ yv, int64_t y_bs, int64_t n,
    int h_in, int h_out) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][kT * kPStr];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][kT * kPStr];
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, l32 = lane % 32, hf = lane / 32;
  const int wm = wave / 2, wn = wave % 2;
  const int tiles_n = (h_out + kT - 1) / kT;
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t m0 = static_cast<int64_t>(t / tiles_n) * kT;
  const int n0 = (t % tiles_n) * kT;
  const int64_t b = blockIdx.y;
  const uint16_t* x = a + b * a_bs;
  const uint16_t* x2 = a2 ? a2 + b * a_bs : nullptr;
  const uint16_t* wb = w + b * w_bs;

  // thread -> (row, 16-byte chunk): 128 rows x 4 chunks, 2 per thread
  uint4 ra[2], rb[2];
  auto load = [&](const uint16_t* xs, int k0) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int u = tid + q * kThreads;
      const int row = u / 4, c = u % 4;
      const int k = k0 + 8 * c;
      ra[q] = (m0 + row < n && k < h_in)
                  ? *reinterpret_cast<const uint4*>(xs + (m0 + row) * h_in + k)
                  : make_uint4(0, 0, 0, 0);
      rb[q] = (n0 + row < h_out && k < h_in)
                  ? *reinterpret_cast<const uint4*>(wb + static_cast<int64_t>(n0 + row) * h_in + k)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int u = tid + q * kThreads;
      const int row = u / 4, c = u % 4;
      *reinterpret_cast<uint4*>(sa[buf] + row * kPStr + 8 * c) = ra[q];
      *reinterpret_cast<uint4*>(sb[buf] + row * kPStr + 8 * c) = rb[q];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = (h_in + kPK - 1) / kPK;
  const int nst = x2 ? 2 * nk : nk;  // stage s < nk: plane a; s >= nk: plane a2
  auto stage_src = [&](int s, const uint16_t*& xs, int& k0) {
    xs = s < nk ? x : x2;
    k0 = (s < nk ? s : s - nk) * kPK;
  };
  {
    const uint16_t* xs;
    int k0;
    stage_src(0, xs, k0);
    load(xs, k0);
  }
  store(0);
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    const int buf = s & 1;
    const bool has_next = s + 1 < nst;
    if (has_next) {
      const uint16_t* xs;
      int k0;
      stage_src(s + 1, xs, k0);
      load(xs, k0);
    }
#pragma unroll
    for (int kk = 0; kk < kPK / 16; ++kk) {
      bf16x8 av[2], bb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        av[i] = *reinterpret_cast<const bf16x8*>(sa[buf] + (wm * 64 + i * 32 + l32) * kPStr +
                                                 16 * kk + 8 * hf);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bb[j] = *reinterpret_cast<const bf16x8*>(sb[buf] + (wn * 64 + j * 32 + l32) * kPStr +
                                                 16 * kk + 8 * hf);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(av[i], bb[j], acc[i][j]);
    }
    if (has_next) store(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int o = n0 + wn * 64 + j * 32 + l32;
      if (o >= h_out) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
        if (m >= n) continue;
        if constexpr (F32OUT)
          static_cast<float*>(yv)[b * y_bs + m * h_out + o] = acc[i][j][r];
        else
          static_cast<uint16_t*>(yv)[b * y_bs + m * h_out + o] = f32_to_bf16_bits(acc[i][j][r]);
      }
    }
  }
}

// fp32 -> two bf16 planes: hi = rne(c), lo = rne(c - hi); hi + lo holds c to
// about 2^-17 relative.
__global__ void split_bf16_kernel(const float* __restrict__ c, uint16_t* __restrict__ hi,
                                  uint16_t* __restrict__ lo, int64_t count) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < count;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const float v = c[i];
    const uint16_t h = f32_to_bf16_bits(v);
    hi[i] = h;
    lo[i] = f32_to_bf16_bits(v - bf16_bits_to_f32(h));
  }
}

}  // namespace

hipError_t launch_gram(const GramParams& p, hipStream_t stream) {
  if (p.batch <= 0) return hipSuccess;
  const int nbp = (p.h + kT - 1) / kT;
  const int nb2 = p.d ? 2 * nbp : nbp;
  const int n_tiles = nb2 * (nb2 + 1) / 2;
  hipLaunchKernelGGL(gram_kernel, dim3(n_tiles, p.batch), dim3(kThreads), 0, stream, p, nbp,
                     n_tiles);
  return hipGetLastError();
}

// Fraction of the compute units busy, averaged over the rounds, when `tiles`
// equal workgroups (one per CU) run on `cus` compute units.
static double round_fill(int64_t tiles, int cus) {
  const int64_t rounds = (tiles + cus - 1) / cus;
  return rounds ? static_cast<double>(tiles) / static_cast<double>(rounds * cus) : 0.0;
}

hipError_t launch_project(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t n, int h_in,
                          int h_out, hipStream_t stream) {
  if (nt_gemm256_supported(h_in)) {
    // Three tilings: 256 x 128, 192 x 256 and 256 x 256 run a FLOP 1, 1.28
    // and 1.41 times as fast (fewer operand bytes and barriers per MFMA;
    // measured at a contraction of 5120) but come in fewer, larger tiles.
    // Take the one whose rate times its fill of the rounds of one tile per CU
    // is highest: e.g. 4680 x 5120 outputs are 760, 500 and 380 tiles on
    // 256 CUs, 99 %, 98 % and 74 % of whole rounds, and 192 x 256 wins.
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorInvalidDevice;
    const int64_t rows256 = (n + 255) / 256, rows192 = (n + 191) / 192;
    const int64_t cols256 = (h_out + 255) / 256, cols128 = (h_out + 127) / 128;
    const double r128 = round_fill(rows256 * cols128, cus);
    const double r192 = 1.28 * round_fill(rows192 * cols256, cus);
    const double r256 = 1.41 * round_fill(rows256 * cols256, cus);
    if (r256 >= r192 && r256 > r128) return launch_g256_bf16(x, w, y, n, h_in, h_out, stream, 256);
    if (r192 > r128) return launch_g256_bf16(x, w, y, n, h_in, h_out, stream, 192);
    return launch_nt_gemm256_bf16(x, w, y, n, h_in, h_out, stream);
  }
  const int64_t tiles = ((n + kT - 1) / kT) * ((h_out + kT - 1) / kT);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(nt_gemm_kernel<false>, dim3(static_cast<unsigned>(tiles)), dim3(kThreads), 0,
                     stream, x, nullptr, 0, w, 0, static_cast<void*>(y), 0, n, h_in, h_out);
  return hipGetLastError();
}

hipError_t launch_split_nt_gemm_f32(const float* c, uint16_t* hi, uint16_t* lo,
                                    const uint16_t* w, float* y, int h, int batch,
                                    hipStream_t stream) {
  const int64_t hh = static_cast<int64_t>(h) * h;
  const int64_t count = hh * batch;
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(split_bf16_kernel, dim3(4096), dim3(256), 0, stream, c, hi, lo, count);
  if (nt_gemm256_supported(h)) return launch_g256_split_f32(hi, lo, w, y, h, batch, stream);
  const int64_t tiles = static_cast<int64_t>((h + kT - 1) / kT) * ((h + kT - 1) / kT);
  hipLaunchKernelGGL(nt_gemm_kernel<true>, dim3(static_cast<unsigned>(tiles), batch),
                     dim3(kThreads), 0, stream, hi, lo, hh, w, hh, static_cast<void*>(y), hh,
                     static_cast<int64_t>(h), h, h);
  return hipGetLastError();
}

}  // namespace ispa
