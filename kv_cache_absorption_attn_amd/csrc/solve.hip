// Ridge-solve pieces, layer scoring, selection and the in-place weight update.
//
// ISPA paper §3.2 (closed-form least-squares absorb at the end of warmup),
// §4.1 (ridge parameter lambda), §3.3 (rank layers by ascending error, the K
// lowest take W_new = W + dW in place).
//
// The blocked Cholesky factors G + lambda I one 128-column block at a time:
// this file holds the diagonal-block factorisation (register-blocked, with
// the inverse of the factor for the GEMM-based panel and triangular solves),
// the probes that decide which layers' solves are refined, and the small
// elementwise pieces; the panel and trailing updates are fp32 MFMA GEMMs.

#include <float.h>

#include "device_common.h"
#include "ispa_internal.h"

namespace ispa {
namespace {

constexpr int kNB = 128;

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
//
// Register-blocked: thread t holds the 8 x 8 block (t / 16, t % 16) of the
// block's lower triangle, first of the factor, then of its inverse (blocks
// above the diagonal stay zero). Each step broadcasts one column of the
// factor (and, for the inverse, one row) through LDS and every thread
// updates its own block in registers: two barriers per column, instead of a
// chain of dependent LDS read-modify-writes per element and column.
__global__ __launch_bounds__(256) void potrf_block_kernel(float* __restrict__ L,
                                                          float* __restrict__ Linv, int h,
                                                          int k0, int nb, int* __restrict__ info,
                                                          int info_first) {
  __shared__ float s_col[kNB];  // a column of the factor below the diagonal
  __shared__ float s_row[kNB];  // a row of the inverse
  __shared__ float s_dg[kNB];   // the diagonal of the factor
  __shared__ int s_fail;
  const int b = blockIdx.x, t = threadIdx.x;
  const int bi = t / 16, bj = t % 16;
  const int i0 = 8 * bi, c0 = 8 * bj;
  const bool lower = bi >= bj;
  float* Lb = L + b * static_cast<int64_t>(h) * h + static_cast<int64_t>(k0) * h + k0;

  float a[8][8];
#pragma unroll
  for (int ii = 0; ii < 8; ++ii)
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) a[ii][cc] = 0.f;
  if (lower && c0 < nb) {
#pragma unroll
    for (int ii = 0; ii < 8; ++ii) {
      const int i = i0 + ii;
      if (i >= nb) continue;
      const float4 lo = *reinterpret_cast<const float4*>(Lb + static_cast<int64_t>(i) * h + c0);
      const float4 hi = *reinterpret_cast<const float4*>(Lb + static_cast<int64_t>(i) * h + c0 + 4);
      const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) a[ii][cc] = (c0 + cc <= i) ? v[cc] : 0.f;
    }
  }
  if (t == 0) s_fail = 0;
  __syncthreads();

  // right-looking factorisation, one column j at a time
  for (int jb = 0; jb < kNB / 8; ++jb) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = 8 * jb + jj;
      if (j >= nb) continue;  // uniform
      if (bi == jb && bj == jb) {
        float d = a[jj][jj];
        if (!(d > 0.f)) {
          if (s_fail == 0) s_fail = j + 1;
          d = 1.f;
        }
        const float r = sqrtf(d);
        a[jj][jj] = r;
        s_dg[j] = r;
      }
      __syncthreads();
      if (bj == jb && bi >= jb) {
        const float inv = 1.f / s_dg[j];
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const int i = i0 + ii;
          if (i > j && i < nb) {
            a[ii][jj] *= inv;
            s_col[i] = a[ii][jj];
          }
        }
      }
      __syncthreads();
      // A(i, c) -= L(i, j) L(c, j) for j < c <= i
      if (lower && i0 + 7 > j) {
        float li[8], lc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          li[e] = s_col[i0 + e];
          lc[e] = s_col[c0 + e];
        }
#pragma unroll
        for (int ii = 0; ii < 8; ++ii)
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) {
            const int i = i0 + ii, c = c0 + cc;
            if (c > j && c <= i && i < nb) a[ii][cc] = fmaf(-li[ii], lc[cc], a[ii][cc]);
          }
      }
    }
  }

  // inverse X = L^-1 by rows: X(k, c) = (delta_kc - sum_{m<k} L(k, m) X(m, c)) / L(k, k),
  // the sums kept per element and updated once row k is final
  float x[8][8];
#pragma unroll
  for (int ii = 0; ii < 8; ++ii)
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) x[ii][cc] = (i0 + ii == c0 + cc && i0 + ii < nb) ? 1.f : 0.f;
  for (int kb = 0; kb < kNB / 8; ++kb) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int k = 8 * kb + kk;
      if (k >= nb) continue;  // uniform
      if (bi == kb && bj <= kb) {
        const float dinv = 1.f / s_dg[k];
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
          const int c = c0 + cc;
          if (c <= k) {
            x[kk][cc] *= dinv;
            s_row[c] = x[kk][cc];
          }
        }
      }
      if (bj == kb && bi >= kb) {
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const int i = i0 + ii;
          if (i > k && i < nb) s_col[i] = a[ii][kk];
        }
      }
      __syncthreads();
      // X(i, c) -= L(i, k) X(k, c) for i > k, c <= k
      if (lower && i0 + 7 > k && c0 <= k) {
        float li[8], xr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          li[e] = s_col[i0 + e];
          xr[e] = s_row[c0 + e];
        }
#pragma unroll
        for (int ii = 0; ii < 8; ++ii)
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) {
            const int i = i0 + ii, c = c0 + cc;
            if (i > k && i < nb && c <= k) x[ii][cc] = fmaf(-li[ii], xr[cc], x[ii][cc]);
          }
      }
      __syncthreads();
    }
  }

  float* Lib = Linv + b * static_cast<int64_t>(h) * kNB + static_cast<int64_t>(k0) * kNB;
  if (c0 < nb) {
#pragma unroll
    for (int ii = 0; ii < 8; ++ii) {
      const int i = i0 + ii;
      if (i >= nb) continue;
      if (lower) {
#pragma unroll
        for (int cc = 0; cc < 8; ++cc)
          if (c0 + cc <= i) Lb[static_cast<int64_t>(i) * h + c0 + cc] = a[ii][cc];
      }
      *reinterpret_cast<float4*>(Lib + i * kNB + c0) =
          make_float4(x[ii][0], x[ii][1], x[ii][2], x[ii][3]);
      *reinterpret_cast<float4*>(Lib + i * kNB + c0 + 4) =
          make_float4(x[ii][4], x[ii][5], x[ii][6], x[ii][7]);
    }
  }
  if (t == 0) {
    if (info_first) info[b] = s_fail ? k0 + s_fail : 0;
    else if (s_fail && info[b] == 0) info[b] = k0 + s_fail;
  }
}

// y += x elementwise (float4; the refinement's Y = Y0 + correction).
__global__ void add_inplace_kernel(float* __restrict__ y, const float* __restrict__ x,
                                   int64_t n4, const int* __restrict__ mask) {
  const int b = blockIdx.y;
  if (mask && !mask[b]) return;
  float4* yb = reinterpret_cast<float4*>(y) + b * n4;
  const float4* xb = reinterpret_cast<const float4*>(x) + b * n4;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n4;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    float4 a = yb[i];
    const float4 c = xb[i];
    a.x += c.x; a.y += c.y; a.z += c.z; a.w += c.w;
    yb[i] = a;
  }
}

// ------------------------------------------------------------ refinement probes
// Eight probe columns z_j (j < 8) with entries +-1: bit j of a hash of the row
// index (a 32-bit integer mix; any fixed pseudo-random signs serve).
__device__ __forceinline__ uint32_t probe_bits(uint32_t o) {
  uint32_t x = o * 0x9E3779B1u + 0x7F4A7C15u;
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

// Q[b][k][j] = sum_o Wo[b][o][k] z_j(o): one thread per k, the signs of a
// 256-row chunk of o staged in LDS.
__global__ __launch_bounds__(256) void probe_wz_kernel(const uint16_t* __restrict__ Wo,
                                                       double* __restrict__ Q, int h) {
  __shared__ uint32_t zs[256];
  const int b = blockIdx.y;
  const int k = blockIdx.x * 256 + threadIdx.x;
  const uint16_t* W = Wo + static_cast<int64_t>(b) * h * h;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int o0 = 0; o0 < h; o0 += 256) {
    __syncthreads();
    zs[threadIdx.x] = probe_bits(static_cast<uint32_t>(o0 + threadIdx.x));
    __syncthreads();
    const int n = h - o0 < 256 ? h - o0 : 256;
    if (k < h) {
      for (int t = 0; t < n; ++t) {
        const float w = bf16_bits_to_f32(W[static_cast<int64_t>(o0 + t) * h + k]);
        const uint32_t z = zs[t];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += ((z >> j) & 1u) ? w : -w;
      }
    }
  }
  if (k < h) {
    double* q = Q + (static_cast<int64_t>(b) * h + k) * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = acc[j];
  }
}

// Y[b] = X[b] Q[b] (X fp32 h x h, Q fp64 h x 8), fp64 accumulation. A block of
// 256 threads owns 64 rows; thread t takes row t % 64 and probes 2 (t / 64)
// and 2 (t / 64) + 1; 64 x 64 tiles of X and 64 rows of Q go through LDS.
__global__ __launch_bounds__(256) void mv8_f64_kernel(const float* __restrict__ X,
                                                      const double* __restrict__ Q,
                                                      double* __restrict__ Y, int h) {
  __shared__ float xs[64][65];
  __shared__ double qs[64][8];
  const int b = blockIdx.y;
  const int row0 = blockIdx.x * 64;
  const int t = threadIdx.x, r = t % 64, p = t / 64;
  const float* Xb = X + static_cast<int64_t>(b) * h * h;
  const double* Qb = Q + static_cast<int64_t>(b) * h * 8;
  double a0 = 0.0, a1 = 0.0;
  for (int k0 = 0; k0 < h; k0 += 64) {
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = t + 256 * e, rr = idx / 16, c4 = (idx % 16) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (row0 + rr < h && k0 + c4 < h)
        v = *reinterpret_cast<const float4*>(Xb + static_cast<int64_t>(row0 + rr) * h + k0 + c4);
      xs[rr][c4] = v.x;
      xs[rr][c4 + 1] = v.y;
      xs[rr][c4 + 2] = v.z;
      xs[rr][c4 + 3] = v.w;
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int idx = t + 256 * e, kk = idx / 8, j = idx % 8;
      qs[kk][j] = k0 + kk < h ? Qb[static_cast<int64_t>(k0 + kk) * 8 + j] : 0.0;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 64; ++kk) {
      const double x = xs[r][kk];
      a0 = fma(x, qs[kk][2 * p], a0);
      a1 = fma(x, qs[kk][2 * p + 1], a1);
    }
  }
  if (row0 + r < h) {
    double* y = Y + (static_cast<int64_t>(b) * h + row0 + r) * 8 + 2 * p;
    y[0] = a0;
    y[1] = a1;
  }
}

// R[b] = A[b] - T[b] - lam B[b] (h x 8), rounded to fp32 for the solve.
__global__ void probe_resid_kernel(const double* __restrict__ A, const double* __restrict__ T,
                                   const double* __restrict__ B, double lam, float* __restrict__ R,
                                   int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    R[i] = static_cast<float>(A[i] - T[i] - lam * B[i]);
}

// flag[b] = !(||E[b]|| <= tol ||B[b]||): one block per layer, fixed-order sums.
__global__ __launch_bounds__(256) void probe_flag_kernel(const float* __restrict__ E,
                                                         const double* __restrict__ B, double tol,
                                                         int* __restrict__ flag, int h) {
  __shared__ double se[256], sb[256];
  const int b = blockIdx.x;
  const int64_t n = static_cast<int64_t>(h) * 8;
  const float* e = E + b * n;
  const double* v = B + b * n;
  double ae = 0.0, ab = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) {
    const double x = e[i];
    ae = fma(x, x, ae);
    ab = fma(v[i], v[i], ab);
  }
  se[threadIdx.x] = ae;
  sb[threadIdx.x] = ab;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      se[threadIdx.x] += se[threadIdx.x + s];
      sb[threadIdx.x] += sb[threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) flag[b] = (se[0] <= tol * tol * sb[0]) ? 0 : 1;
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
// The first form equals the direct residual ||X (W + dW) - Z W||^2 at the
// ridge optimum; away from it the two differ by tr(dW^T r) with r = C W -
// (G + lambda I) dW, which the refined solve keeps at the level of fp32
// rounding. What remains is the rounding of the fp32 traces, of the order
// of 2^-24 sqrt(h) of ||Z W||^2; a near-exact fit can fall below zero by
// that much, and a squared norm is clamped at zero.
__global__ __launch_bounds__(256) void score_finalize_kernel(const ScoreParams p, int nrb) {
  extern __shared__ double key[];
  const int L = p.n_layers;
  for (int l = threadIdx.x; l < L; l += blockDim.x) {
    double s[kNPart] = {0, 0, 0, 0, 0};
    for (int rb = 0; rb < nrb; ++rb)
      for (int q = 0; q < kNPart; ++q) s[q] += p.partial[(static_cast<int64_t>(l) * nrb + rb) * kNPart + q];
    const double tew = s[0], tgw = s[1], tcw = s[2], tdb = s[3], dd = s[4];
    double ea = tew - tdb - static_cast<double>(p.lam) * dd;
    if (ea < 0.0) ea = 0.0;
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
  hipLaunchKernelGGL(potrf_block_kernel, dim3(batch), dim3(256), 0, stream, L, Linv, h, k0, nb,
                     info, info_first);
  return hipGetLastError();
}

hipError_t launch_add_inplace(float* y, const float* x, int64_t n, int batch,
                              const int* layer_mask, hipStream_t stream) {
  const int64_t n4 = n / 4;
  if (n4 == 0 || batch <= 0) return hipSuccess;
  const int64_t blocks = (n4 + 255) / 256;
  hipLaunchKernelGGL(add_inplace_kernel,
                     dim3(static_cast<unsigned>(blocks < 1024 ? blocks : 1024), batch), dim3(256),
                     0, stream, y, x, n4, layer_mask);
  return hipGetLastError();
}

hipError_t launch_probe_wz(const uint16_t* Wo, double* Q, int h, int batch, hipStream_t stream) {
  if (h <= 0 || batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(probe_wz_kernel, dim3((h + 255) / 256, batch), dim3(256), 0, stream, Wo, Q,
                     h);
  return hipGetLastError();
}

hipError_t launch_mv8_f64(const float* X, const double* Q, double* Y, int h, int batch,
                          hipStream_t stream) {
  if (h <= 0 || batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(mv8_f64_kernel, dim3((h + 63) / 64, batch), dim3(256), 0, stream, X, Q, Y, h);
  return hipGetLastError();
}

hipError_t launch_probe_resid(const double* A, const double* T, const double* B, double lam,
                              float* R, int h, int batch, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(h) * 8 * batch;
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(probe_resid_kernel, dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)),
                     dim3(256), 0, stream, A, T, B, lam, R, n);
  return hipGetLastError();
}

hipError_t launch_probe_flag(const float* E, const double* B, double tol, int* flag, int h,
                             int batch, hipStream_t stream) {
  if (h <= 0 || batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(probe_flag_kernel, dim3(batch), dim3(256), 0, stream, E, B, tol, flag, h);
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
