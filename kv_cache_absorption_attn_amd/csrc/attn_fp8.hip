// Operand preparation of the E4M3 decomposable attention (the quantized
// attention in the spirit of SageAttention, which the ISPA paper, "Towards
// Memory-Efficient Autoregressive Video Generation via Instance-Specific
// Parametric Absorption", §3.4
// cites; §4.4 runs ISPA with 8-bit quantization): per-(token, head) query
// codes with the LSE smoothing shift, per-(64-key tile, head) codes of the
// smoothed keys, and the key mean used as the smoothing vector.
//
// Codes are OCP E4M3 ("fn"): for a block with absmax a, scale = a / 448
// and code = nearest E4M3 value of fp32(v * (448 / a)), ties to even
// (v_cvt_pk_fp8_f32); a block of zeros gets scale 0 and zero codes. The
// smoothed key is formed in fp32 as k - mu from the bf16 values. All of
// these decisions are taken in fp32 with correctly rounded divisions.

#include "device_common.h"
#include "ispa_internal.h"

namespace ispa {
namespace {

constexpr int kHd = 128;                 // head_dim of the E4M3 path
constexpr float kE4M3Max = 448.f;

__device__ __forceinline__ float wave_max(float m) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  return m;
}

__device__ __forceinline__ float wave_sum(float s) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  return s;
}

// Two E4M3 codes of fp32 values, low byte first.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}

// One wave per (token, head) row of 128 values, 4 rows per workgroup: lane
// l holds channels 2l, 2l + 1. Rows are token-major (row = token * n_heads +
// head), so a workgroup reads 4 consecutive head slices of one token.
__global__ __launch_bounds__(256) void quantize_queries_kernel(
    const uint16_t* __restrict__ q, int64_t rows, int n_heads, int64_t n_q,
    const uint16_t* __restrict__ mu, float sm_scale, uint8_t* __restrict__ q8,
    float* __restrict__ qsc, float* __restrict__ qmu) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / 64;
  if (row >= rows) return;
  const int lane = threadIdx.x % 64;
  const int64_t tok = row / n_heads;
  const int head = static_cast<int>(row % n_heads);
  const uint32_t w = *reinterpret_cast<const uint32_t*>(q + row * kHd + 2 * lane);
  const float x0 = __uint_as_float(w << 16), x1 = __uint_as_float(w & 0xFFFF0000u);
  const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
  const float inv = amax > 0.f ? kE4M3Max / amax : 0.f;
  reinterpret_cast<uint16_t*>(q8 + row * kHd)[lane] =
      static_cast<uint16_t>(e4m3x2(x0 * inv, x1 * inv));
  float dot = 0.f;
  if (mu) {
    const uint32_t m = *reinterpret_cast<const uint32_t*>(mu + head * kHd + 2 * lane);
    dot = wave_sum(x0 * __uint_as_float(m << 16) + x1 * __uint_as_float(m & 0xFFFF0000u));
  }
  if (lane == 0) {
    qsc[head * n_q + tok] = amax > 0.f ? amax / kE4M3Max : 0.f;
    if (qmu) qmu[head * n_q + tok] = sm_scale * dot;
  }
}

// One workgroup per (64-key tile, head) of a segment: thread t takes key row
// t / 4 of the tile and channels 32 (t % 4) .. + 31. Rows past the segment
// end take no part (the last tile may be partial).
__global__ __launch_bounds__(256) void quantize_key_tiles_kernel(
    const uint16_t* __restrict__ k, int64_t n, int n_heads, const uint16_t* __restrict__ mu,
    uint8_t* __restrict__ k8, float* __restrict__ ksc) {
  __shared__ float red[4];
  const int tile = blockIdx.x / n_heads;
  const int head = blockIdx.x % n_heads;
  const int t = threadIdx.x;
  const int64_t key = static_cast<int64_t>(tile) * 64 + t / 4;
  const int c0 = 32 * (t % 4);
  const bool live = key < n;
  float r[32];
  float m = 0.f;
  if (live) {
    const uint16_t* src = k + (key * n_heads + head) * kHd + c0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + 8 * j);
      uint4 mv = make_uint4(0, 0, 0, 0);
      if (mu) mv = *reinterpret_cast<const uint4*>(mu + head * kHd + c0 + 8 * j);
      const uint32_t kw[4] = {v.x, v.y, v.z, v.w};
      const uint32_t mw[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        r[8 * j + 2 * i] = __uint_as_float(kw[i] << 16) - __uint_as_float(mw[i] << 16);
        r[8 * j + 2 * i + 1] =
            __uint_as_float(kw[i] & 0xFFFF0000u) - __uint_as_float(mw[i] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(r[i]));
  }
  m = wave_max(m);
  if (t % 64 == 0) red[t / 64] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = amax > 0.f ? kE4M3Max / amax : 0.f;
  if (t == 0) ksc[blockIdx.x] = amax > 0.f ? amax / kE4M3Max : 0.f;
  if (!live) return;
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    out[i] = e4m3x2(r[4 * i] * inv, r[4 * i + 1] * inv) |
             (e4m3x2(r[4 * i + 2] * inv, r[4 * i + 3] * inv) << 16);
  uint4* dst = reinterpret_cast<uint4*>(k8 + (key * n_heads + head) * kHd + c0);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
}

// Key mean, pass 1: column sums of the flattened key rows [n, C] (C =
// n_heads * 128) over the rows r = s, s + S, ... of the three segments taken
// in order, in fp32; thread = 8 consecutive columns, grid (C / 2048
// rounded up, S). Partial sums go to part[s][C] (a fixed order: the result
// does not depend on scheduling).
__global__ __launch_bounds__(256) void key_sum_partial_kernel(KeySegs segs, int64_t cols,
                                                              float* __restrict__ part) {
  const int64_t c = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (c >= cols) return;
  const int s = blockIdx.y, S = gridDim.y;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int g = 0; g < 3; ++g) {
    const uint16_t* base = segs.k[g];
    for (int64_t r = s; r < segs.n[g]; r += S) {
      const uint4 v = *reinterpret_cast<const uint4*>(base + r * cols + c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += __uint_as_float(w[i] << 16);
        acc[2 * i + 1] += __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
  }
  float* dst = part + static_cast<int64_t>(s) * cols + c;
#pragma unroll
  for (int i = 0; i < 8; ++i) dst[i] = acc[i];
}

// Pass 2: mean = (sum of the S partials, in order, in fp64) / n, rounded to
// bf16.
__global__ __launch_bounds__(256) void key_mean_finalize_kernel(const float* __restrict__ part,
                                                                int S, int64_t cols, int64_t n,
                                                                uint16_t* __restrict__ mu) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (c >= cols) return;
  double acc = 0.0;
  for (int s = 0; s < S; ++s) acc += part[static_cast<int64_t>(s) * cols + c];
  mu[c] = f32_to_bf16_bits(static_cast<float>(acc / static_cast<double>(n)));
}

}  // namespace

hipError_t launch_quantize_queries_fp8(const uint16_t* q, int64_t n_q, int n_heads,
                                       const uint16_t* mu, float sm_scale, uint8_t* q8,
                                       float* qsc, float* qmu, hipStream_t stream) {
  const int64_t rows = n_q * n_heads;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_queries_kernel, dim3(static_cast<unsigned>((rows + 3) / 4)),
                     dim3(256), 0, stream, q, rows, n_heads, n_q, mu, sm_scale, q8, qsc, qmu);
  return hipGetLastError();
}

int64_t key_tiles(int64_t n) { return (n + 63) / 64; }

hipError_t launch_quantize_key_tiles_fp8(const uint16_t* k, int64_t n, int n_heads,
                                         const uint16_t* mu, uint8_t* k8, float* ksc,
                                         hipStream_t stream) {
  const int64_t blocks = key_tiles(n) * n_heads;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_key_tiles_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, k, n, n_heads, mu, k8, ksc);
  return hipGetLastError();
}

int key_mean_splits() { return 128; }

hipError_t launch_key_mean(const KeySegs& segs, int n_heads, float* part, uint16_t* mu,
                           hipStream_t stream) {
  const int64_t cols = static_cast<int64_t>(n_heads) * kHd;
  const int64_t n = segs.n[0] + segs.n[1] + segs.n[2];
  const int S = key_mean_splits();
  hipLaunchKernelGGL(key_sum_partial_kernel,
                     dim3(static_cast<unsigned>((cols / 8 + 255) / 256), S), dim3(256), 0, stream,
                     segs, cols, part);
  hipLaunchKernelGGL(key_mean_finalize_kernel, dim3(static_cast<unsigned>((cols + 255) / 256)),
                     dim3(256), 0, stream, part, S, cols, n, mu);
  return hipGetLastError();
}

}  // namespace ispa
