// Untracked direct-to-LDS loads for kernels that stage operands through a
// multi-slot LDS ring (the NT GEMM).
#ifndef ISPA_LDS_DMA_ASM_H_
#define ISPA_LDS_DMA_ASM_H_

#include "device_common.h"

namespace ispa {

// Buffer descriptor of a raw (untyped) range from `base`: the same four
// dwords as raw_rsrc, as plain SGPRs for the asm load below.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 desc_of(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 d;
  d.x = static_cast<uint32_t>(a);
  d.y = static_cast<uint32_t>(a >> 32) & 0xFFFFu;  // stride 0
  d.z = 0x7fffffffu;                               // no practical range limit
  d.w = 0x00020000u;                               // 32-bit data format
  return d;
}

// Direct-to-LDS 16-byte load (lane l's 16 bytes at voff + soff land at
// lds + 16 l) written in asm, so the compiler does not track it. With the
// builtin, the wait-count pass of a multi-slot LDS ring keeps the loads of
// earlier ring turns pending at the loop head and drains every load in
// flight there once per turn. Kernels using this helper wait explicitly
// (vmcnt before the barrier that publishes a stage) and keep their LDS reads
// below those waits with memory clobbers. No VGPR is written by the load (its data
// goes to LDS); one wait state separates the M0 write from its use.
__device__ __forceinline__ void dma16_asm(const u32x4& d, uint16_t* lds, uint32_t voff, int soff) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ISPA_LDS(void, lds))));
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(m0v), "v"(voff), "s"(d), "s"(soff)
      : "memory", "m0");
}

}  // namespace ispa

#endif  // ISPA_LDS_DMA_ASM_H_
