// Warmup statistics and the L-layer projection on CDNA4 bf16 matrix cores.
//
// Gram accumulation (ISPA paper §3.1 item 2: the accumulated dual-stream
// activations are the basis of the weight adaption): for X = O_local and
// D = O_full - O_local of one warmup step, G += X^T X, C += X^T D, E += D^T D,
// in fp32. Treating Y = [X | D] as one [n_tok, 2h] matrix, every needed block
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
constexpr int kTStr = kTok + 8;  // LDS row stride (bf16) of a Y^T tile

// One operand of the Gram: a 128-feature block of Y staged as Y^T[f][t].
// Thread -> (token group of 4, 8-feature chunk): 4 row loads of 16 bytes,
// written as 8 transposed 8-byte chunks.
struct GramLoader {
  uint4 r[4];
  __device__ void load(const uint16_t* base, int h, int fvalid, int64_t t0, int64_t n_tok,
                       int tid) {
    const int tg = tid % 16, fc = tid / 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t t = t0 + 4 * tg + j;
      if (t < n_tok && 8 * fc < fvalid) {
        r[j] = *reinterpret_cast<const uint4*>(base + t * h + 8 * fc);
      } else {
        r[j] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ void store(uint16_t* S, int tid) const {
    const int tg = tid % 16, fc = tid / 16;
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r[0]);
    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r[1]);
    const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r[2]);
    const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r[3]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int wi = e >> 1;
      uint2 v;
      if ((e & 1) == 0) {
        v.x = pack_lo16(w0[wi], w1[wi]);
        v.y = pack_lo16(w2[wi], w3[wi]);
      } else {
        v.x = pack_hi16(w0[wi], w1[wi]);
        v.y = pack_hi16(w2[wi], w3[wi]);
      }
      *reinterpret_cast<uint2*>(S + (8 * fc + e) * kTStr + 4 * tg) = v;
    }
  }
};

__global__ __launch_bounds__(kThreads, 2) void gram_kernel(const GramParams p, int nbp,
                                                            int n_tiles) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][2][kT * kTStr];

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, l32 = lane % 32, hf = lane / 32;
  const int wm = wave / 2, wn = wave % 2;
  const int b = blockIdx.y;

  // tile id -> (bi, bj), bi <= bj, over the 2*nbp block rows of Y^T Y
  int idx = xcd_remap(blockIdx.x, n_tiles);
  const int nb2 = 2 * nbp;
  int bi = 0;
  while (idx >= nb2 - bi) {
    idx -= nb2 - bi;
    ++bi;
  }
  const int bj = bi + idx;

  const int h = p.h;
  const int64_t hh = static_cast<int64_t>(h) * h;
  const uint16_t* xb = p.x + b * p.n_tok * h;
  const uint16_t* db = p.d + b * p.n_tok * h;
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
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nst = static_cast<int>((p.n_tok + kTok - 1) / kTok);
  if (nst > 0) {
    li.load(srci, h, fvi, 0, p.n_tok, tid);
    lj.load(srcj, h, fvj, 0, p.n_tok, tid);
    li.store(smem[0][0], tid);
    lj.store(smem[0][1], tid);
  }
  __syncthreads();

  for (int s = 0; s < nst; ++s) {
    const int buf = s & 1;
    const bool has_next = s + 1 < nst;
    if (has_next) {
      li.load(srci, h, fvi, static_cast<int64_t>(s + 1) * kTok, p.n_tok, tid);
      lj.load(srcj, h, fvj, static_cast<int64_t>(s + 1) * kTok, p.n_tok, tid);
    }
    const uint16_t* si = smem[buf][0];
    const uint16_t* sj = smem[buf][1];
#pragma unroll
    for (int kk = 0; kk < kTok / 16; ++kk) {
      bf16x8 a[2], bb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(si + (wm * 64 + i * 32 + l32) * kTStr +
                                                16 * kk + 8 * hf);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bb[j] = *reinterpret_cast<const bf16x8*>(sj + (wn * 64 + j * 32 + l32) * kTStr +
                                                 16 * kk + 8 * hf);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(a[i], bb[j], acc[i][j]);
    }
    if (has_next) {
      li.store(smem[buf ^ 1][0], tid);
      lj.store(smem[buf ^ 1][1], tid);
    }
    __syncthreads();
  }

  // dest(fi0 + m, fj0 + n) (+)= acc; mirror tile for off-diagonal G / E tiles.
  const bool mirror = (i_is_d == j_is_d) && bi != bj;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = wn * 64 + j * 32 + l32;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int m0 = wm * 64 + i * 32 + 8 * g + 4 * hf;
        if (n < fvj) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (m0 + r < fvi) {
              float* c = dest + static_cast<int64_t>(fi0 + m0 + r) * h + fj0 + n;
              const float v = acc[i][j][4 * g + r];
              *c = p.zero_first ? v : *c + v;
            }
          }
          if (mirror && m0 + 4 <= fvi) {
            float4* c = reinterpret_cast<float4*>(dest + static_cast<int64_t>(fj0 + n) * h +
                                                  fi0 + m0);
            float4 v = make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1],
                                   acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
            if (!p.zero_first) {
              const float4 o = *c;
              v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
            }
            *c = v;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- projection
constexpr int kPK = 32;           // k per stage
constexpr int kPStr = kPK + 8;    // LDS row stride (bf16)

__global__ __launch_bounds__(kThreads, 2) void project_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ w,
                                                               uint16_t* __restrict__ y,
                                                               int64_t n, int h_in, int h_out) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][kT * kPStr];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][kT * kPStr];
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, l32 = lane % 32, hf = lane / 32;
  const int wm = wave / 2, wn = wave % 2;
  const int tiles_n = (h_out + kT - 1) / kT;
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t m0 = static_cast<int64_t>(t / tiles_n) * kT;
  const int n0 = (t % tiles_n) * kT;

  // thread -> (row, 16-byte chunk): 128 rows x 4 chunks, 2 per thread
  uint4 ra[2], rb[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int u = tid + q * kThreads;
      const int row = u / 4, c = u % 4;
      const int k = k0 + 8 * c;
      ra[q] = (m0 + row < n && k < h_in)
                  ? *reinterpret_cast<const uint4*>(x + (m0 + row) * h_in + k)
                  : make_uint4(0, 0, 0, 0);
      rb[q] = (n0 + row < h_out && k < h_in)
                  ? *reinterpret_cast<const uint4*>(w + static_cast<int64_t>(n0 + row) * h_in + k)
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

  const int nst = (h_in + kPK - 1) / kPK;
  load(0);
  store(0);
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    const int buf = s & 1;
    const bool has_next = s + 1 < nst;
    if (has_next) load((s + 1) * kPK);
#pragma unroll
    for (int kk = 0; kk < kPK / 16; ++kk) {
      bf16x8 a[2], bb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(sa[buf] + (wm * 64 + i * 32 + l32) * kPStr +
                                                16 * kk + 8 * hf);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bb[j] = *reinterpret_cast<const bf16x8*>(sb[buf] + (wn * 64 + j * 32 + l32) * kPStr +
                                                 16 * kk + 8 * hf);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(a[i], bb[j], acc[i][j]);
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
        if (m < n) y[m * h_out + o] = f32_to_bf16_bits(acc[i][j][r]);
      }
    }
  }
}

}  // namespace

hipError_t launch_gram(const GramParams& p, hipStream_t stream) {
  const int nbp = (p.h + kT - 1) / kT;
  const int nb2 = 2 * nbp;
  const int n_tiles = nb2 * (nb2 + 1) / 2;
  if (p.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(gram_kernel, dim3(n_tiles, p.batch), dim3(kThreads), 0, stream, p, nbp,
                     n_tiles);
  return hipGetLastError();
}

hipError_t launch_project(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t n, int h_in,
                          int h_out, hipStream_t stream) {
  const int64_t tiles = ((n + kT - 1) / kT) * ((h_out + kT - 1) / kT);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(project_kernel, dim3(static_cast<unsigned>(tiles)), dim3(kThreads), 0,
                     stream, x, w, y, n, h_in, h_out);
  return hipGetLastError();
}

}  // namespace ispa
