// Device-side helpers shared by the ISPA HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ispa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 <-> fp32 on raw 16-bit storage.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (gfx950 lowers the cast to
// v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16_bits(lo)) |
         (static_cast<uint32_t>(f32_to_bf16_bits(hi)) << 16);
}

// Interleave 16-bit halves of two words: (lo16(a), lo16(b)) and (hi16(a), hi16(b)).
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// 32x32x16 bf16 MFMA, fp32 accumulate. Operand lane layout used throughout:
// lane l holds A[m = l%32][k-slot j] and B[k-slot j][n = l%32] for j = 0..7 of
// k-half l/32; the result lane l, register i holds D[m = 8*(i/4) + 4*(l/32) +
// (i%4)][n = l%32].
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 32x32x2 fp32 MFMA: lane l holds A[m = l%32][k = l/32], B[k = l/32][n = l%32].
__device__ __forceinline__ f32x16 mfma32x32x2f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// LDS tiles of 16-bit elements with rows of D elements (D = 128: 256-byte
// rows; D = 64: 128-byte rows) store the 16-byte chunk c of row r at chunk
// position c ^ lds_swz<D>(r). With the 64-bank LDS this spreads 16
// consecutive rows reading one logical chunk (16-byte operand reads, 16 lanes
// per pass) and 4 consecutive rows x 4 adjacent chunks (transposing 8-byte
// reads, 32 lanes per pass) over distinct banks.
template <int D>
__device__ __forceinline__ int lds_swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return ((r & 2) << 1) | ((r >> 2) & 3);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define ISPA_LDS(T, ptr) ((__attribute__((address_space(3))) T*)(ptr))

// Element (row, col) of a swizzled LDS tile with rows of D elements.
template <int D>
__device__ __forceinline__ const uint16_t* swz_addr(const uint16_t* base, int row, int col) {
  return base + row * D + 8 * ((col >> 3) ^ lds_swz<D>(row)) + (col & 7);
}

// MFMA operand whose contraction index runs along the rows of a swizzled
// LDS tile (rows = contraction index, columns = the operand's m or n index):
// lane l receives the 8 elements (rows r(j), column col0 + l%32), j = 0..7,
// with r(j) = row0 + 8*(j/4) + 4*(l/32) + (j%4), by two transposing reads
// (ds_read_b64_tr_b16: within each 16-lane group, lane i gets element i%4 of
// the rows supplied by lanes i/4, i/4+4, i/4+8, i/4+12).
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* base, int row0, int col0, int lane) {
  const int g = lane / 16, i = lane % 16;
  const int r = row0 + 4 * (g / 2) + i / 4;
  const int c = col0 + 16 * (g % 2) + 4 * (i % 4);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(ISPA_LDS(s16x4, swz_addr<D>(base, r, c)));
  const s16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16(ISPA_LDS(s16x4, swz_addr<D>(base, r + 8, c)));
  typedef __bf16 bf16x4_local __attribute__((ext_vector_type(4)));
  return __builtin_shufflevector(__builtin_bit_cast(bf16x4_local, lo),
                                 __builtin_bit_cast(bf16x4_local, hi), 0, 1, 2, 3, 4, 5, 6, 7);
}

// Lane offsets (elements) of the two transposing reads of tr_operand for
// operand columns col0.. of a swizzled tile, for row0 = 0. The swizzle only
// depends on row % 16, so for any row0 that is a multiple of 16 the reads are
// at base + row0 * D + off: the offsets are computed once and every k-step
// only adds a compile-time immediate.
struct TrOff {
  int lo, hi;
};
template <int D>
__device__ __forceinline__ TrOff tr_offsets(int col0, int lane) {
  const int g = lane / 16, i = lane % 16;
  const int r = 4 * (g / 2) + i / 4;
  const int c = col0 + 16 * (g % 2) + 4 * (i % 4);
  TrOff o;
  o.lo = r * D + 8 * ((c >> 3) ^ lds_swz<D>(r)) + (c & 7);
  o.hi = (r + 8) * D + 8 * ((c >> 3) ^ lds_swz<D>(r + 8)) + (c & 7);
  return o;
}

// tr_operand with precomputed lane offsets; row0 % 16 == 0.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand_at(const uint16_t* base, int row0, TrOff o) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(ISPA_LDS(s16x4, base + row0 * D + o.lo));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(ISPA_LDS(s16x4, base + row0 * D + o.hi));
  typedef __bf16 bf16x4_local __attribute__((ext_vector_type(4)));
  return __builtin_shufflevector(__builtin_bit_cast(bf16x4_local, lo),
                                 __builtin_bit_cast(bf16x4_local, hi), 0, 1, 2, 3, 4, 5, 6, 7);
}

// Buffer resource for raw (untyped) loads from `base` with no practical range
// limit (callers issue in-bounds offsets only); the dword-3 value selects a
// 32-bit data format, without which untyped loads on this family read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}

// Direct-to-LDS 16-byte load: lane l's 16 bytes at byte offset `voff` from the
// resource base land at lds + 16 l. The buffer form is used rather than the
// global one: the compiler books a global LDS load as an LDS access of unknown
// order, after which every wait for an LDS read becomes a wait for all of
// them (lgkmcnt(0)), which defeats reading MFMA operands ahead.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, ISPA_LDS(void, lds), 16, voff, 0, 0, 0);
}

// Workgroups are dispatched round-robin over the 8 XCDs of an MI355X. Remap
// the hardware block id so that consecutive logical work items land on the
// same XCD (and share its L2): logical id = start(xcd) + bid / 8.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int per = total / 8, rem = total % 8;
  const int xcd = bid % 8, slot = bid / 8;
  return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

}  // namespace ispa
