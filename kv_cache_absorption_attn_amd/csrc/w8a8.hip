// W8A8 output projection (the ISPA paper, "Towards Memory-Efficient
// Autoregressive Video Generation via Instance-Specific Parametric
// Absorption", §4.4, "Compatibility with Post-Training Quantization": 8-bit
// weights and activations for the linear layers; for an
// L-layer the update is folded in first, W_new = W + dW, then quantized).
// Format: OCP 8-bit floating point E4M3 ("fn": bias 7, no infinities,
// largest finite 448). Each row (an output channel of W, a token of X) gets
// its own scale absmax / 448; codes are the nearest E4M3 values of
// value * (448 / absmax), ties to even, formed in fp32 (the hardware
// conversion rounds to nearest even, and no scaled value exceeds 448 by more
// than an fp32 rounding, far inside the saturation threshold of 464). The
// product runs on the E4M3 matrix cores (nt_gemm.hip) with the two scales
// applied in its epilogue.

#include "device_common.h"
#include "ispa_internal.h"

namespace ispa {
namespace {

constexpr int kQThreads = 256;

// One workgroup per row: absmax, then the scaled codes, 8 values a thread
// and step (k % 8 == 0).
__global__ __launch_bounds__(kQThreads) void quantize_rows_kernel(const uint16_t* __restrict__ a,
                                                                  int k,
                                                                  uint8_t* __restrict__ q,
                                                                  float* __restrict__ scale) {
  __shared__ float red[kQThreads / 64];
  const int64_t r = blockIdx.x;
  const uint16_t* row = a + r * k;
  float m = 0.f;
  for (int c = threadIdx.x * 8; c < k; c += kQThreads * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m = fmaxf(m, fabsf(__uint_as_float(w[i] << 16)));
      m = fmaxf(m, fabsf(__uint_as_float(w[i] & 0xFFFF0000u)));
    }
  }
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = m;
  __syncthreads();
  float amax = red[0];
#pragma unroll
  for (int i = 1; i < kQThreads / 64; ++i) amax = fmaxf(amax, red[i]);
  // correctly rounded fp32 divisions (the compiler's default for '/')
  const float inv = amax > 0.f ? 448.f / amax : 0.f;
  if (threadIdx.x == 0) scale[r] = amax > 0.f ? amax / 448.f : 0.f;
  uint8_t* qr = q + r * k;
  for (int c = threadIdx.x * 8; c < k; c += kQThreads * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float x0 = __uint_as_float(w[2 * i] << 16) * inv;
      const float x1 = __uint_as_float(w[2 * i] & 0xFFFF0000u) * inv;
      const float x2 = __uint_as_float(w[2 * i + 1] << 16) * inv;
      const float x3 = __uint_as_float(w[2 * i + 1] & 0xFFFF0000u) * inv;
      int p = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
      p = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, p, true);
      out[i] = static_cast<uint32_t>(p);
    }
    *reinterpret_cast<uint2*>(qr + c) = make_uint2(out[0], out[1]);
  }
}

}  // namespace

hipError_t launch_quantize_rows_fp8(const uint16_t* a, int64_t rows, int k, uint8_t* q,
                                    float* scale, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3(static_cast<unsigned>(rows)), dim3(kQThreads), 0,
                     stream, a, k, q, scale);
  return hipGetLastError();
}

}  // namespace ispa
