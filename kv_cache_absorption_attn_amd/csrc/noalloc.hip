// Allocation-free variant of the W8A8 output projection, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc). It runs the kernels of
// ispa_project_w8a8 (per-token E4M3 quantization, then the E4M3 NT GEMM) with
// the quantized tokens staged in a fixed device array of this library
// instead of a caller workspace.
//
// The array is a file-scope __device__ variable: each GPU the library runs on
// holds its own copy, at its own address, until the process ends. Host code
// never passes the variable's name to a kernel (on the host that name is a
// stand-in, not a device address): on the first call on a device, with that
// device current, its address is looked up with hipGetSymbolAddress and kept
// per device. Every call on one GPU shares that GPU's copy, so calls that
// overlap on one GPU (different streams, different host threads without
// ordering) race on it. Nothing in it has to start at zero: the quantization
// writes every code and scale that the product then reads.

#include <mutex>
#include <stdint.h>

#include "ispa.h"
#include "ispa_internal.h"

namespace {

constexpr size_t kCodeBytes = static_cast<size_t>(ISPA_NOALLOC_MAX_CODE_BYTES);
constexpr size_t kScaleBytes = static_cast<size_t>(ISPA_NOALLOC_MAX_TOKENS) * sizeof(float);
constexpr size_t kScratchBytes = kCodeBytes + kScaleBytes;
constexpr int kMaxDevices = 64;

}  // namespace

// [codes: n * h_in bytes | scales: n fp32] of the current call.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The current device's copy of the scratch array (looked up once per device).
int scratch_of_current_device(uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ISPA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return ISPA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return ISPA_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return ISPA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int ispa_project_w8a8_noalloc(const void* x, const void* wq, const float* w_scale,
                                         void* y, int64_t n, int h_in, int h_out, void* stream) {
  if (!x || !wq || !w_scale || !y) return ISPA_ERR_NULL;
  if (n < 0 || h_in < 1 || h_out < 1 || n > INT32_MAX) return ISPA_ERR_SHAPE;
  if (h_in % 64 != 0 || h_out % 8 != 0) return ISPA_ERR_UNSUPPORTED;
  if (n > ISPA_NOALLOC_MAX_TOKENS ||
      static_cast<uint64_t>(n) * static_cast<uint64_t>(h_in) > kCodeBytes)
    return ISPA_ERR_SCRATCH;
  if (!aligned16(x) || !aligned16(wq) || !aligned16(w_scale) || !aligned16(y))
    return ISPA_ERR_ALIGN;
  if (n == 0) return ISPA_OK;
  uint8_t* base = nullptr;
  const int st = scratch_of_current_device(&base);
  if (st != ISPA_OK) return st;
  uint8_t* xq = base;
  float* sx = reinterpret_cast<float*>(base + kCodeBytes);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (ispa::launch_quantize_rows_fp8(static_cast<const uint16_t*>(x), n, h_in, xq, sx, s) !=
      hipSuccess)
    return ISPA_ERR_HIP;
  return ispa::launch_nt_gemm256_fp8(xq, sx, static_cast<const uint8_t*>(wq), w_scale,
                                     static_cast<uint16_t*>(y), n, h_in, h_out, s) == hipSuccess
             ? ISPA_OK
             : ISPA_ERR_HIP;
}
