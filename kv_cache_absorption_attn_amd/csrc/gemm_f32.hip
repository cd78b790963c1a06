// Batched fp32 GEMM on CDNA4 matrix cores (v_mfma_f32_32x32x2_f32), the
// building block of the closed-form ridge solve (blocked Cholesky, panel and
// trailing updates, triangular solves, C W and W W^T products).
//
// C[b](m, n) = alpha * sum_k A[b](m, k) B[b](k, n) + beta * C[b](m, n)
//
// Tile 128 x 128 per workgroup, k-stage 16, 4 waves of 64 x 64 (2 x 2 MFMA
// blocks of 32 x 32). Operands are staged k-major in LDS (As[k][m], Bs[k][n])
// from either storage order, converting bf16 operands to fp32 on the way,
// through two register sets, so that a stage's loads are issued two stages
// before its MFMAs. At most 128 VGPRs and 34 KB of LDS per workgroup keep
// four workgroups (four waves a SIMD) on a CU: the kernel lives on that
// occupancy (k-stages of 32, two workgroups a CU, ran 0.75x; three a CU
// 0.9x).
// The whole k range of an output tile is consumed before its epilogue writes,
// so a GEMM whose single tile row (M <= 128) or tile column (N <= 128) covers
// the operand region it overwrites may run in place.

#include <type_traits>

#include "device_common.h"
#include "ispa_internal.h"

namespace ispa {
namespace {

constexpr int kTM = 128, kTN = 128, kTK = 16;
constexpr int kPad = 4;
constexpr int kLd = kTM + kPad;
constexpr int kThreads = 256;

template <bool BF16>
struct Elt;
template <>
struct Elt<false> {
  static constexpr int kVec = 4;
  __device__ static void load(const void* base, int64_t off, float* out) {
    const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
};
template <>
struct Elt<true> {
  static constexpr int kVec = 8;
  __device__ static void load(const void* base, int64_t off, float* out) {
    const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};

// Stage one operand tile (rows = the M or N dimension, 128 of them; k = 16)
// into LDS as S[k][row]. KC: the k index is the contiguous one in memory.
// Element (row, k) of the operand sits at base[row * s_row + k * s_k].
template <bool KC, bool BF16>
struct TileLoader {
  static constexpr int V = Elt<BF16>::kVec;
  static constexpr int kUnits = kTM * kTK / V;            // vectors per tile
  static constexpr int kPerThread = (kUnits + kThreads - 1) / kThreads;
  float r[kPerThread][V];
  bool ok[kPerThread];

  __device__ void load(const void* base, int64_t s_row, int64_t s_k, int row0, int rows,
                       int k0, int kdim, int tid) {
#pragma unroll
    for (int p = 0; p < kPerThread; ++p) {
      const int u = tid + p * kThreads;
      int row, k;
      if (KC) {  // vectors run along k: kTK / V vectors per row
        row = u / (kTK / V);
        k = (u % (kTK / V)) * V;
      } else {   // vectors run along rows: kTM / V vectors per k
        k = u / (kTM / V);
        row = (u % (kTM / V)) * V;
      }
      const bool in = u < kUnits && (row0 + row) < rows && (k0 + k) < kdim;
      ok[p] = in;
      if (in) {
        const int64_t off = static_cast<int64_t>(row0 + row) * s_row +
                            static_cast<int64_t>(k0 + k) * s_k;
        Elt<BF16>::load(base, off, r[p]);
      }
    }
  }

  __device__ void store(float* S, int tid) const {
#pragma unroll
    for (int p = 0; p < kPerThread; ++p) {
      const int u = tid + p * kThreads;
      if (u >= kUnits) continue;
      int row, k;
      if (KC) {
        row = u / (kTK / V);
        k = (u % (kTK / V)) * V;
#pragma unroll
        for (int e = 0; e < V; ++e) S[(k + e) * kLd + row] = ok[p] ? r[p][e] : 0.f;
      } else {
        k = u / (kTM / V);
        row = (u % (kTM / V)) * V;
#pragma unroll
        for (int e = 0; e < V; ++e) S[k * kLd + row + e] = ok[p] ? r[p][e] : 0.f;
      }
    }
  }
};

template <bool AKC, bool ABF, bool BKC, bool BBF>
__global__ __launch_bounds__(kThreads, 4) void gemm_f32_kernel(const GemmF32Params p) {
  __shared__ __attribute__((aligned(16))) float As[2][kTK * kLd];
  __shared__ __attribute__((aligned(16))) float Bs[2][kTK * kLd];

  const int tiles_n = (p.N + kTN - 1) / kTN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  if (p.tri && tm < tn) return;
  const int b = blockIdx.y;
  if (p.layer_mask && !p.layer_mask[b]) return;
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, l32 = lane % 32, hf = lane / 32;
  const int wm = wave / 2, wn = wave % 2;

  const char* Abase = static_cast<const char*>(p.A) + b * p.a_batch * (ABF ? 2 : 4);
  const char* Bbase = static_cast<const char*>(p.B) + b * p.b_batch * (BBF ? 2 : 4);
  float* Cb = p.Cm + b * p.c_batch;
  // A(m, k) = Abase[m * a_s0 + k * a_s1]; B(k, n) = Bbase[k * b_s0 + n * b_s1]
  const int64_t a_srow = p.a_s0, a_sk = p.a_s1;
  const int64_t b_srow = p.b_s1, b_sk = p.b_s0;

  // two register sets of operand tiles: stage ks + 2 is loaded while stage
  // ks is multiplied and stage ks + 1 waits in the other set for its store,
  // so a load has two stages of MFMA work to arrive
  TileLoader<AKC, ABF> la[2];
  TileLoader<BKC, BBF> lb[2];
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = (p.K + kTK - 1) / kTK;
  la[0].load(Abase, a_srow, a_sk, tm * kTM, p.M, 0, p.K, tid);
  lb[0].load(Bbase, b_srow, b_sk, tn * kTN, p.N, 0, p.K, tid);
  if (nk > 1) {
    la[1].load(Abase, a_srow, a_sk, tm * kTM, p.M, kTK, p.K, tid);
    lb[1].load(Bbase, b_srow, b_sk, tn * kTN, p.N, kTK, p.K, tid);
  }
  la[0].store(As[0], tid);
  lb[0].store(Bs[0], tid);
  __syncthreads();

  // stage ks from LDS slot S = ks % 2; register set S held it and takes stage
  // ks + 2, set S ^ 1 holds stage ks + 1 and goes to the other slot, which
  // every wave finished reading before the previous barrier
  auto step = [&](int ks, auto s_c) __attribute__((always_inline)) {
    constexpr int S = decltype(s_c)::value;
    if (ks + 2 < nk) {
      la[S].load(Abase, a_srow, a_sk, tm * kTM, p.M, (ks + 2) * kTK, p.K, tid);
      lb[S].load(Bbase, b_srow, b_sk, tn * kTN, p.N, (ks + 2) * kTK, p.K, tid);
    }
    const float* as = As[S];
    const float* bs = Bs[S];
#pragma unroll
    for (int kk = 0; kk < kTK / 2; ++kk) {
      const int k = 2 * kk + hf;
      float a[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = as[k * kLd + wm * 64 + i * 32 + l32];
#pragma unroll
      for (int j = 0; j < 2; ++j) bv[j] = bs[k * kLd + wn * 64 + j * 32 + l32];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x2f32(a[i], bv[j], acc[i][j]);
    }
    if (ks + 1 < nk) {
      la[S ^ 1].store(As[S ^ 1], tid);
      lb[S ^ 1].store(Bs[S ^ 1], tid);
    }
    __syncthreads();
  };
  for (int ks = 0; ks < nk; ks += 2) {
    step(ks, std::integral_constant<int, 0>{});
    if (ks + 1 < nk) step(ks + 1, std::integral_constant<int, 1>{});
  }

#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = tn * kTN + wn * 64 + j * 32 + l32;
      if (n >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = tm * kTM + wm * 64 + i * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
        if (m >= p.M) continue;
        float* c = Cb + static_cast<int64_t>(m) * p.ldc + n;
        float v = p.alpha * acc[i][j][r];
        if (p.beta != 0.f) v += p.beta * *c;
        *c = v;
      }
    }
  }
}

// Residual of the ridge system with fp64 accumulation, for one step of
// iterative refinement of its fp32 solution (ISPA paper §3.2, closed-form
// least squares; §4.1, ridge lambda):
//   S[b] = C[b] - lambda Y[b] - G[b] Y[b]        (all h x h fp32, row-major)
// The fp32 inputs are widened to fp64 on the way from LDS to the fp64 matrix
// cores (v_mfma_f64_16x16x4f64), so each product is exact and the sum over k
// is rounded at fp64 precision; only the small result is rounded to fp32.
// The refinement needs this: the residual is a near-cancellation of C and
// G Y, and an fp32-accumulated one carries errors of 2^-24 |G| |Y| that the
// solve amplifies by up to 1/lambda.
//
// Tile 128 x 128 per workgroup, k-stage 16 (the fp32 tile loader above),
// 4 waves of 64 x 64 = 4 x 4 blocks of 16 x 16. MFMA lane layout: lane l
// holds A[m = l % 16][k = l / 16] and B[k = l / 16][n = l % 16]; result
// register r of lane l is D[m = 4 r + l / 16][n = l % 16] (one row per
// 64-bit register, the lane groups interleaved).
typedef double f64x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads, 2) void ridge_resid_f64_kernel(const RidgeResidParams p) {
  __shared__ __attribute__((aligned(16))) float As[2][kTK * kLd];
  __shared__ __attribute__((aligned(16))) float Bs[2][kTK * kLd];
  const int h = p.h;
  const int tiles_n = (h + kTN - 1) / kTN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int64_t hh = static_cast<int64_t>(h) * h;
  const int64_t b = blockIdx.y;
  if (p.layer_mask && !p.layer_mask[b]) return;
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, l16 = lane % 16, q = lane / 16;
  const int wm = wave / 2, wn = wave % 2;
  const float* G = p.G + b * hh;
  const float* Y = p.Y + b * hh;

  // A(m, k) = G[m][k] (k contiguous); B(k, n) = Y[k][n] (n contiguous)
  TileLoader<true, false> la;
  TileLoader<false, false> lb;
  f64x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};

  const int nk = (h + kTK - 1) / kTK;
  la.load(G, h, 1, tm * kTM, h, 0, h, tid);
  lb.load(Y, 1, h, tn * kTN, h, 0, h, tid);
  la.store(As[0], tid);
  lb.store(Bs[0], tid);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    const bool has_next = ks + 1 < nk;
    if (has_next) {
      la.load(G, h, 1, tm * kTM, h, (ks + 1) * kTK, h, tid);
      lb.load(Y, 1, h, tn * kTN, h, (ks + 1) * kTK, h, tid);
    }
    const float* as = As[buf];
    const float* bs = Bs[buf];
#pragma unroll
    for (int kk = 0; kk < kTK / 4; ++kk) {
      const int k = 4 * kk + q;
      double a[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = static_cast<double>(as[k * kLd + wm * 64 + i * 16 + l16]);
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = static_cast<double>(bs[k * kLd + wn * 64 + j * 16 + l16]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (has_next) {
      la.store(As[buf ^ 1], tid);
      lb.store(Bs[buf ^ 1], tid);
    }
    __syncthreads();
  }

  const float* C = p.C + b * hh;
  float* S = p.S + b * hh;
  const double lam = p.lam;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = tn * kTN + wn * 64 + j * 16 + l16;
      if (n >= h) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = tm * kTM + wm * 64 + i * 16 + 4 * r + q;
        if (m >= h) continue;
        const int64_t e = static_cast<int64_t>(m) * h + n;
        const double v = static_cast<double>(C[e]) - lam * static_cast<double>(Y[e]) - acc[i][j][r];
        S[e] = static_cast<float>(v);
      }
    }
}

}  // namespace

hipError_t launch_ridge_resid_f64(const RidgeResidParams& p, hipStream_t stream) {
  if (p.h <= 0 || p.batch <= 0) return hipSuccess;
  const int t = (p.h + kTM - 1) / kTM;
  hipLaunchKernelGGL(ridge_resid_f64_kernel, dim3(t * t, p.batch), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmF32Params& p, hipStream_t stream) {
  if (p.M <= 0 || p.N <= 0 || p.batch <= 0) return hipSuccess;
  const int tiles = ((p.M + kTM - 1) / kTM) * ((p.N + kTN - 1) / kTN);
  const dim3 grid(tiles, p.batch);
  const bool akc = p.a_s1 == 1, bkc = p.b_s0 == 1;
#define ISPA_GEMM_CASE(AKC, ABF, BKC, BBF)                                                  \
  if (akc == AKC && (p.a_bf16 != 0) == ABF && bkc == BKC && (p.b_bf16 != 0) == BBF) {       \
    hipLaunchKernelGGL((gemm_f32_kernel<AKC, ABF, BKC, BBF>), grid, dim3(kThreads), 0, stream, \
                       p);                                                                  \
    return hipGetLastError();                                                               \
  }
  ISPA_GEMM_CASE(true, false, true, false)    // panel: A row-major, B = Linv^T
  ISPA_GEMM_CASE(true, false, false, false)   // trsm fwd update / diag solve
  ISPA_GEMM_CASE(false, false, false, false)  // trsm bwd update / diag solve
  ISPA_GEMM_CASE(true, false, true, true)     // B = C W (W bf16, torch layout)
  ISPA_GEMM_CASE(false, true, false, true)    // P = W W^T (bf16 torch layout)
#undef ISPA_GEMM_CASE
  return hipErrorInvalidValue;
}

}  // namespace ispa
