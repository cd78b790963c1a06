// Ridge-solve pieces, layer scoring, selection and the in-place weight update.
//
// ISPA paper §3.2 (closed-form least-squares absorb at the end of warmup),
// §4.1 (ridge parameter lambda), §3.3 (rank layers by ascending error, the K
// lowest take W_new = W + dW in place).
//
// The blocked Cholesky factors G + lambda I one 128-column block at a time:
// this file holds the diagonal-block factorisation (in LDS, with the inverse
// of the factor for the GEMM-based panel and triangular solves); the panel
// and trailing updates are fp32 MFMA GEMMs.

#include <float.h>

#include "device_common.h"
#include "ispa_internal.h"

namespace ispa {
namespace {

constexpr int kNB = 128;
constexpr int kLdsLd = kNB + 1;

__global__ void copy_add_diag_kernel(const float* __restrict__ G, float* __restrict__ L, int h,
                                     float lam) {
  const int64_t hh = static_cast<int64_t>(h) * h;
  const int b = blockIdx.y;
  const int64_t i4 = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i4 >= hh) return;
  float4 v = *reinterpret_cast<const float4*>(G + b * hh + i4);
  const int64_t r = i4 / h, c0 = i4 % h;
  if (r >= c0 && r < c0 + 4) {
    const int k = static_cast<int>(r - c0);
    if (k == 0) v.x += lam;
    if (k == 1) v.y += lam;
    if (k == 2) v.z += lam;
    if (k == 3) v.w += lam;
  }
  *reinterpret_cast<float4*>(L + b * hh + i4) = v;
}

// Factor the diagonal block L[k0:k0+nb, k0:k0+nb] (already holding the
// trailing-updated values) in place and write its inverse to Linv ([nb][kNB]
// row-major). info[b] gets the 1-based global index of the first
// non-positive pivot (0 when the block, and all earlier ones, were fine); a
// failing pivot is replaced by 1 so the factorisation still runs to the end
// with finite values.
__global__ __launch_bounds__(256) void potrf_block_kernel(float* __restrict__ L,
                                                          float* __restrict__ Linv, int h,
                                                          int k0, int nb, int* __restrict__ info,
                                                          int info_first) {
  extern __shared__ float lds[];
  float* A = lds;                   // [kNB][kLdsLd]
  float* X = lds + kNB * kLdsLd;    // [kNB][kLdsLd]
  __shared__ float s_inv;
  __shared__ int s_fail;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t hh = static_cast<int64_t>(h) * h;
  float* Lb = L + b * hh;

  for (int e = tid; e < nb * nb; e += blockDim.x) {
    const int i = e / nb, j = e % nb;
    A[i * kLdsLd + j] = (j <= i) ? Lb[static_cast<int64_t>(k0 + i) * h + k0 + j] : 0.f;
  }
  if (tid == 0) s_fail = 0;
  __syncthreads();

  const int ti = tid / 16, tc = tid % 16;
  for (int j = 0; j < nb; ++j) {
    if (tid == 0) {
      float d = A[j * kLdsLd + j];
      if (!(d > 0.f)) {
        if (s_fail == 0) s_fail = j + 1;
        d = 1.f;
      }
      const float r = sqrtf(d);
      A[j * kLdsLd + j] = r;
      s_inv = 1.f / r;
    }
    __syncthreads();
    const float inv = s_inv;
    for (int i = j + 1 + tid; i < nb; i += blockDim.x) A[i * kLdsLd + j] *= inv;
    __syncthreads();
    // trailing update of the lower triangle: A[i][c] -= A[i][j] A[c][j], j < c <= i
    const int first = j + 1;
    for (int i = first + ((ti - first) % 16 + 16) % 16; i < nb; i += 16) {
      const float aij = A[i * kLdsLd + j];
      for (int c = first + ((tc - first) % 16 + 16) % 16; c <= i; c += 16) {
        A[i * kLdsLd + c] -= aij * A[c * kLdsLd + j];
      }
    }
    __syncthreads();
  }

  // inverse of the lower-triangular factor, one column per thread
  if (tid < nb) {
    const int c = tid;
    for (int i = 0; i < nb; ++i) {
      float v;
      if (i < c) {
        v = 0.f;
      } else if (i == c) {
        v = 1.f / A[c * kLdsLd + c];
      } else {
        float s = 0.f;
        for (int k = c; k < i; ++k) s = fmaf(A[i * kLdsLd + k], X[k * kLdsLd + c], s);
        v = -s / A[i * kLdsLd + i];
      }
      X[i * kLdsLd + c] = v;
    }
  }
  __syncthreads();

  float* Lib = Linv + b * static_cast<int64_t>(h) * kNB + static_cast<int64_t>(k0) * kNB;
  for (int e = tid; e < nb * nb; e += blockDim.x) {
    const int i = e / nb, j = e % nb;
    if (j <= i) Lb[static_cast<int64_t>(k0 + i) * h + k0 + j] = A[i * kLdsLd + j];
    Lib[i * kNB + j] = X[i * kLdsLd + j];
  }
  if (tid == 0) {
    if (info_first) info[b] = s_fail ? k0 + s_fail : 0;
    else if (s_fail && info[b] == 0) info[b] = k0 + s_fail;
  }
}

// dst[b](j, i) = src[b](i, j) for an h x h matrix, 32 x 32 tiles via LDS.
__global__ void transpose_kernel(const float* __restrict__ src, float* __restrict__ dst, int h) {
  __shared__ float t[32][33];
  const int64_t hh = static_cast<int64_t>(h) * h;
  const int b = blockIdx.z;
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
  const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;  // 256 threads: 32 x 8
  for (int r = ty; r < 32; r += 8) {
    const int i = i0 + r, j = j0 + tx;
    if (i < h && j < h) t[r][tx] = src[b * hh + static_cast<int64_t>(i) * h + j];
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int j = j0 + r, i = i0 + tx;
    if (i < h && j < h) dst[b * hh + static_cast<int64_t>(j) * h + i] = t[tx][r];
  }
}

__device__ __forceinline__ double block_sum(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  double s = 0.0;
  if (threadIdx.x == 0)
    for (int i = 0; i < static_cast<int>(blockDim.x / 64); ++i) s += red[i];
  return s;
}

// Per (layer, 128-row block) partial sums, fp64:
//  0: sum E.P   1: sum G.P   (P = W W^T symmetric: lower 128-tiles weighted 2,
//                             diagonal tiles weighted 1; only those are read)
//  2: sum Bt.Wt (= tr(W^T C W))   3: sum dWt.Bt (= tr(dW^T C W))   4: sum dWt^2
constexpr int kNPart = 5;
__global__ __launch_bounds__(256) void score_reduce_kernel(const ScoreParams p,
                                                           const float* __restrict__ P,
                                                           const float* __restrict__ Bt,
                                                           int nrb) {
  __shared__ double red[4];
  const int l = blockIdx.y, rb = blockIdx.x, h = p.h;
  const int64_t hh = static_cast<int64_t>(h) * h;
  const int r0 = rb * kNB, r1 = min(h, r0 + kNB);
  const int cdiag = r0, cend = min(h, r0 + kNB);
  const float* E = p.E + l * hh;
  const float* G = p.G + l * hh;
  const float* Pl = P + l * hh;
  const float* Btl = Bt + l * hh;
  const float* dW = p.dW + l * hh;
  const uint16_t* W = p.Wo + l * hh;
  double sep = 0.0, sgp = 0.0, sbw = 0.0, sdb = 0.0, sdd = 0.0;
  for (int r = r0; r < r1; ++r) {
    const int64_t row = static_cast<int64_t>(r) * h;
    for (int c = threadIdx.x; c < cend; c += blockDim.x) {
      const double wgt = c < cdiag ? 2.0 : 1.0;
      const double pv = static_cast<double>(Pl[row + c]) * wgt;
      sep += static_cast<double>(E[row + c]) * pv;
      sgp += static_cast<double>(G[row + c]) * pv;
    }
    for (int c = threadIdx.x; c < h; c += blockDim.x) {
      const double bt = Btl[row + c];
      const double dw = dW[row + c];
      sbw += bt * static_cast<double>(bf16_bits_to_f32(W[row + c]));
      sdb += dw * bt;
      sdd += dw * dw;
    }
  }
  double* out = p.partial + (static_cast<int64_t>(l) * nrb + rb) * kNPart;
  double v;
  v = block_sum(sep, red); if (threadIdx.x == 0) out[0] = v;
  v = block_sum(sgp, red); if (threadIdx.x == 0) out[1] = v;
  v = block_sum(sbw, red); if (threadIdx.x == 0) out[2] = v;
  v = block_sum(sdb, red); if (threadIdx.x == 0) out[3] = v;
  v = block_sum(sdd, red); if (threadIdx.x == 0) out[4] = v;
}

// eps_abs = tr(W^T E W) - tr(dW^T C W) - lambda ||dW||^2
// eps_rel = eps_abs / ||Z W||^2,  ||Z W||^2 = tr(W^T (G + C + C^T + E) W)
// then a stable ascending ranking; the first K valid layers are selected.
__global__ __launch_bounds__(256) void score_finalize_kernel(const ScoreParams p, int nrb) {
  extern __shared__ double key[];
  const int L = p.n_layers;
  for (int l = threadIdx.x; l < L; l += blockDim.x) {
    double s[kNPart] = {0, 0, 0, 0, 0};
    for (int rb = 0; rb < nrb; ++rb)
      for (int q = 0; q < kNPart; ++q) s[q] += p.partial[(static_cast<int64_t>(l) * nrb + rb) * kNPart + q];
    const double tew = s[0], tgw = s[1], tcw = s[2], tdb = s[3], dd = s[4];
    double ea = tew - tdb - static_cast<double>(p.lam) * dd;
    const double den = tgw + 2.0 * tcw + tew;
    double er = den > 0.0 ? ea / den : (ea == 0.0 ? 0.0 : INFINITY);
    const bool bad = (p.info && p.info[l] != 0) || isnan(ea) || isnan(er);
    if (bad) {
      ea = INFINITY;
      er = INFINITY;
    }
    p.eps_abs[l] = ea;
    p.eps_rel[l] = er;
    key[l] = er;
  }
  __syncthreads();
  for (int l = threadIdx.x; l < L; l += blockDim.x) {
    const double kl = key[l];
    int rank = 0;
    for (int j = 0; j < L; ++j) {
      const double kj = key[j];
      rank += (kj < kl) || (kj == kl && j < l);
    }
    p.selected[l] = (rank < p.K && kl < INFINITY) ? 1 : 0;
  }
}

// Wo[l] <- bf16(Wo[l] + dW[l]) for selected layers, correctly rounded: the
// fp32 sum carries its exact rounding error (two-sum), which breaks the tie
// when the fp32 sum sits exactly halfway between two bf16 values.
__device__ __forceinline__ uint16_t add_round_bf16(float a, float b) {
  const float s = a + b;
  const float bb = s - a;
  const float err = (a - (s - bb)) + (b - bb);
  const uint32_t bits = __float_as_uint(s);
  if ((bits & 0xFFFFu) == 0x8000u && err != 0.f && (bits & 0x7F800000u) != 0x7F800000u) {
    const bool up_mag = (err > 0.f) == (s > 0.f);
    return static_cast<uint16_t>((bits >> 16) + (up_mag ? 1u : 0u));
  }
  if ((bits & 0x7F800000u) == 0x7F800000u) return static_cast<uint16_t>(bits >> 16);
  const uint32_t r = bits + 0x7FFFu + ((bits >> 16) & 1u);
  return static_cast<uint16_t>(r >> 16);
}

__global__ void apply_dw_kernel(const int* __restrict__ selected, const float* __restrict__ dW,
                                uint16_t* __restrict__ Wo, int64_t hh) {
  const int l = blockIdx.y;
  if (!selected[l]) return;
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i >= hh) return;
  const float4 d = *reinterpret_cast<const float4*>(dW + l * hh + i);
  uint2* wp = reinterpret_cast<uint2*>(Wo + l * hh + i);
  const uint2 w = *wp;
  uint2 o;
  o.x = static_cast<uint32_t>(add_round_bf16(__uint_as_float(w.x << 16), d.x)) |
        (static_cast<uint32_t>(add_round_bf16(__uint_as_float(w.x & 0xFFFF0000u), d.y)) << 16);
  o.y = static_cast<uint32_t>(add_round_bf16(__uint_as_float(w.y << 16), d.z)) |
        (static_cast<uint32_t>(add_round_bf16(__uint_as_float(w.y & 0xFFFF0000u), d.w)) << 16);
  *wp = o;
}

// ---------------------------------------------------------------- drift score
// (event-triggered recalibration, ISPA paper §3.3 last paragraph)

// Identity of order h in each [h, h] fp32 matrix of the batch (grid.y).
__global__ void identity_kernel(float* __restrict__ M, int h, int64_t hh) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= hh) return;
  M[blockIdx.y * hh + i] = (i / h == i % h) ? 1.f : 0.f;
}

// Per (matrix, block of rows) fp64 partial sums of squares of a rows x cols
// fp32 matrix (row stride ld), in a fixed order.
__global__ __launch_bounds__(256) void sumsq_kernel(const float* __restrict__ A, int rows,
                                                    int cols, int64_t ld, int64_t mat_stride,
                                                    int rows_per_block,
                                                    double* __restrict__ partial) {
  __shared__ double red[4];
  const float* Al = A + blockIdx.y * mat_stride;
  const int r0 = blockIdx.x * rows_per_block;
  const int r1 = min(rows, r0 + rows_per_block);
  double s = 0.0;
  for (int r = r0; r < r1; ++r)
    for (int c = threadIdx.x; c < cols; c += blockDim.x) {
      const double v = Al[static_cast<int64_t>(r) * ld + c];
      s += v * v;
    }
  const double t = block_sum(s, red);
  if (threadIdx.x == 0) partial[static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x] = t;
}

// With S = the summed squares of matrix l:
//   reference (ref == null): out[l] = (h - lambda S) / n_warm, the expected
//     leverage tr((G + lambda I)^{-1} G) / N with S = ||L^{-1}||_F^2 =
//     tr((G + lambda I)^{-1});
//   score: out[l] = (S / n_sample) / ref[l], S = sum of the sample's
//     leverages ||L^{-1} x^T||^2.
__global__ void drift_finalize_kernel(const double* __restrict__ partial, int nblk, int n_layers,
                                      double h, double lam, double n_div,
                                      const double* __restrict__ ref, double* __restrict__ out) {
  for (int l = threadIdx.x; l < n_layers; l += blockDim.x) {
    double S = 0.0;
    for (int i = 0; i < nblk; ++i) S += partial[static_cast<int64_t>(l) * nblk + i];
    out[l] = ref ? (S / n_div) / ref[l] : (h - lam * S) / n_div;
  }
}

}  // namespace

hipError_t launch_identity(float* M, int h, int batch, hipStream_t stream) {
  const int64_t hh = static_cast<int64_t>(h) * h;
  hipLaunchKernelGGL(identity_kernel, dim3(static_cast<unsigned>((hh + 255) / 256), batch),
                     dim3(256), 0, stream, M, h, hh);
  return hipGetLastError();
}

int drift_partial_count(int rows) { return (rows + kNB - 1) / kNB; }

hipError_t launch_drift_sum(const float* A, int rows, int cols, int64_t ld, int64_t mat_stride,
                            int batch, double* partial, double h, double lam, double n_div,
                            const double* ref, double* out, hipStream_t stream) {
  const int nblk = drift_partial_count(rows);
  hipLaunchKernelGGL(sumsq_kernel, dim3(nblk, batch), dim3(256), 0, stream, A, rows, cols, ld,
                     mat_stride, kNB, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(drift_finalize_kernel, dim3(1), dim3(256), 0, stream, partial, nblk, batch,
                     h, lam, n_div, ref, out);
  return hipGetLastError();
}

hipError_t launch_copy_add_diag(const float* G, float* L, int h, int batch, float lam,
                                hipStream_t stream) {
  const int64_t hh = static_cast<int64_t>(h) * h;
  const int64_t blocks = (hh / 4 + 255) / 256;
  hipLaunchKernelGGL(copy_add_diag_kernel, dim3(static_cast<unsigned>(blocks), batch), dim3(256),
                     0, stream, G, L, h, lam);
  return hipGetLastError();
}

hipError_t launch_potrf_block(float* L, float* Linv, int h, int k0, int nb, int batch, int* info,
                              int info_first, hipStream_t stream) {
  const size_t lds = 2 * kNB * kLdsLd * sizeof(float);
  // set on every call (cheap): no process-wide state, valid for any device
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(potrf_block_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(potrf_block_kernel, dim3(batch), dim3(256), lds, stream, L, Linv, h, k0, nb,
                     info, info_first);
  return hipGetLastError();
}

hipError_t launch_transpose(const float* src, float* dst, int h, int batch, hipStream_t stream) {
  const int t = (h + 31) / 32;
  hipLaunchKernelGGL(transpose_kernel, dim3(t, t, batch), dim3(256), 0, stream, src, dst, h);
  return hipGetLastError();
}

size_t layer_score_partial_count(int n_layers, int h) {
  return static_cast<size_t>(n_layers) * ((h + kNB - 1) / kNB) * kNPart;
}

hipError_t launch_score(const ScoreParams& p, const float* P, const float* Bt,
                        hipStream_t stream) {
  const int nrb = (p.h + kNB - 1) / kNB;
  hipLaunchKernelGGL(score_reduce_kernel, dim3(nrb, p.n_layers), dim3(256), 0, stream, p, P, Bt,
                     nrb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(score_finalize_kernel, dim3(1), dim3(256), p.n_layers * sizeof(double),
                     stream, p, nrb);
  return hipGetLastError();
}

hipError_t launch_apply_dw(int n_layers, int h, const int* selected, const float* dW,
                           uint16_t* Wo, hipStream_t stream) {
  const int64_t hh = static_cast<int64_t>(h) * h;
  const int64_t blocks = (hh / 4 + 255) / 256;
  hipLaunchKernelGGL(apply_dw_kernel, dim3(static_cast<unsigned>(blocks), n_layers), dim3(256),
                     0, stream, selected, dW, Wo, hh);
  return hipGetLastError();
}

}  // namespace ispa
