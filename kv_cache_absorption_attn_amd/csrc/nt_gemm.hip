// NT GEMM on bf16 matrix cores, fp32 accumulate, for the L-layer output
// projection Y = X W^T (ISPA paper §3.1 item 3) and the C W_o product of the
// closed-form absorb (§3.2): Y[m][o] = sum_k A[m][k] W[o][k], both operands
// k-contiguous. Used when the contraction length is a multiple of 32. An
// E4M3 instance (operands as 8-bit codes with per-row scales, §4.4 W8A8)
// runs the same ring with 64 k per stage.
//
// Workgroup tile 256 (m) x 128 (o), 8 waves of 64 x 64 (2 x 2 blocks of
// 32x32x16 MFMAs, 64 accumulators a lane). Arithmetic intensity
// 2*256*128*32 FLOP per 24 KB staged = 85 FLOP/B, against 64 for 128 x 128
// tiles, so the L2 -> CU operand stream stays well under the CU's load
// bandwidth at the MFMA rate this kernel reaches.
//
// k-stages of 32 go through a 4-slot LDS ring filled by direct-to-LDS buffer
// loads issued three stages ahead: each wave waits for its own loads of the
// stage it is about to read (vmcnt), one barrier per stage publishes them and
// frees the slot that the next issue overwrites. A row's 16-byte chunk c
// (k = 8c .. 8c+7 of the stage) is stored at chunk position c ^ ((r >> 2) & 3)
// of its 64-byte LDS row, so the 16 rows of one quarter-wave's 16-byte
// fragment reads cover all 64 banks once. Rows past the matrix re-load its
// last row (their results are never stored).

#include "device_common.h"
#include "ispa_internal.h"
#include "lds_dma_asm.h"

namespace ispa {
namespace {

constexpr int kBM = 256, kBN = 128, kBK = 32;  // kBK: bf16 k per stage
constexpr int kNtThreads = 512;
constexpr int kRowE = kBK;                 // bf16 elements per LDS row (64 bytes)
constexpr int kGroupM = 8;                 // row tiles per L2 group

__device__ __forceinline__ int chunk_pos(int row, int c) { return c ^ ((row >> 2) & 3); }

// 16 bytes of row `row` (chunk position `pos`) of a stage slot.
__device__ __forceinline__ bf16x8 frag(const uint16_t* slot, int row, int pos) {
  return *reinterpret_cast<const bf16x8*>(slot + row * kRowE + 8 * pos);
}

struct NtArgs {
  const void* a;       // [batch][n, h_in] bf16 (or E4M3 codes)
  const void* a2;      // second plane of A (or null): the contraction runs over both
  int64_t a_bs;        // batch strides in elements
  const void* w;       // [batch][h_out, h_in] bf16 (or E4M3 codes)
  int64_t w_bs;
  void* y;             // [batch][n, h_out], bf16 or fp32
  int64_t y_bs;
  int64_t n;
  int h_in, h_out;
  const float* sx;     // E4M3 operands: per-row scales of A [n] and of W [h_out]
  const float* sw;
};

// The products of a grouped launch; the table travels as the kernel argument.
struct NtGroup {
  NtArgs p[kMaxGroup];
  int start[kMaxGroup + 1];
  int n;
};

typedef int v8i32 __attribute__((ext_vector_type(8)));
typedef int v4i32_t __attribute__((ext_vector_type(4)));

// FP8 = false: bf16 operands, 32 k per stage (2 MFMA k-steps of 16).
// FP8 = true: E4M3 operands, 64 k per stage (one 32x32x64 MFMA k-step, lane
// l holding 32 consecutive k of row l % 32 from k = 32 (l / 32)), and the
// epilogue applies the row and column scales. Either way a stage row is 64
// bytes, so loads, swizzle and LDS layout are the same.
// One workgroup tile: logical tile index t (grouped order) of batch entry b.
template <bool F32OUT, bool FP8>
__device__ __forceinline__ void nt_tile(const NtArgs& p, const int t, const int64_t b) {
  __shared__ __attribute__((aligned(16))) uint16_t sa0[kBM * kRowE], sa1[kBM * kRowE],
      sa2[kBM * kRowE], sa3[kBM * kRowE];
  __shared__ __attribute__((aligned(16))) uint16_t sb0[kBN * kRowE], sb1[kBN * kRowE],
      sb2[kBN * kRowE], sb3[kBN * kRowE];
  constexpr int kEs = FP8 ? 1 : 2;        // operand bytes
  constexpr int kKs = 64 / kEs;           // k per stage

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, l32 = lane % 32, hf = lane / 32;
  const int wm = wave / 2, wn = wave % 2;
  const int tiles_m = static_cast<int>((p.n + kBM - 1) / kBM);
  const int tiles_n = (p.h_out + kBN - 1) / kBN;
  // grouped order: kGroupM row tiles share each column panel of W in L2
  const int per_group = kGroupM * tiles_n;
  const int g = t / per_group, first_m = g * kGroupM;
  const int gm = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
  const int tm = first_m + (t % per_group) % gm, tn = (t % per_group) / gm;
  const int64_t m0 = static_cast<int64_t>(tm) * kBM;
  const int n0 = tn * kBN;

  const int nk = p.h_in / kKs;
  const int nst = p.a2 ? 2 * nk : nk;
  const char* abase = static_cast<const char*>(p.a) + b * p.a_bs * kEs;
  const char* a2base = static_cast<const char*>(p.a2 ? p.a2 : p.a) + b * p.a_bs * kEs;
  const u32x4 ra1 = desc_of(abase);
  const u32x4 ra2 = desc_of(a2base);
  const u32x4 rw = desc_of(static_cast<const char*>(p.w) + b * p.w_bs * kEs);

  // per-lane byte offsets of this wave's loads: A rows wave*32 + 16j + lane/4,
  // B rows wave*16 + lane/4; the stage's k offset goes in the scalar offset
  uint32_t va[2], vb;
  {
    const int p4 = lane % 4;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = wave * 32 + 16 * j + lane / 4;
      int64_t gr = m0 + row;
      if (gr > p.n - 1) gr = p.n - 1;
      va[j] = static_cast<uint32_t>(gr * p.h_in * kEs + 16 * chunk_pos(row, p4));
    }
    const int row = wave * 16 + lane / 4;
    int gr = n0 + row;
    if (gr > p.h_out - 1) gr = p.h_out - 1;
    vb = static_cast<uint32_t>(static_cast<int64_t>(gr) * p.h_in * kEs + 16 * chunk_pos(row, p4));
  }
  auto soff_of = [&](int s) { return (s >= nk ? s - nk : s) * 64; };
  auto issue = [&](int s, uint16_t* da, uint16_t* db) {
    const int soff = soff_of(s);
    const u32x4 r = s >= nk ? ra2 : ra1;
    dma16_asm(r, da + (wave * 32) * kRowE, va[0], soff);
    dma16_asm(r, da + (wave * 32 + 16) * kRowE, va[1], soff);
    dma16_asm(rw, db + (wave * 16) * kRowE, vb, soff);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // fragment rows and the chunk positions this lane reads: bf16, chunk
  // 2 kk + hf of k-step kk; E4M3, chunks 2 hf and 2 hf + 1 (32 bytes)
  int ar[2], br[2], apos[2][2], bpos[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    ar[i] = wm * 64 + i * 32 + l32;
    br[i] = wn * 64 + i * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = FP8 ? 2 * hf + kk : 2 * kk + hf;
      apos[i][kk] = chunk_pos(ar[i], c);
      bpos[i][kk] = chunk_pos(br[i], c);
    }
  }

  if (nst > 0) issue(0, sa0, sb0);
  if (nst > 1) issue(1, sa1, sb1);
  if (nst > 2) issue(2, sa2, sb2);

  // one stage: wait for its data, publish, then the MFMAs of its k (the
  // refill of the slot freed by the previous stage spread between the first
  // four)
  auto stage = [&](int s, const uint16_t* __restrict__ ca, const uint16_t* __restrict__ cb,
                   uint16_t* __restrict__ na, uint16_t* __restrict__ nb)
      __attribute__((always_inline)) {
    if (s + 2 < nst)
      asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else if (s + 1 < nst)
      asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // a plain barrier: __syncthreads() would add a workgroup fence, i.e. a
    // wait for every load in flight, including the two stages issued ahead
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    bf16x8 av[2][2], bv[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        av[kk][i] = frag(ca, ar[i], apos[i][kk]);
        bv[kk][i] = frag(cb, br[i], bpos[i][kk]);
      }
    const bool refill = s + 3 < nst;
    const int soff = soff_of(s + 3);
    const u32x4 rsa = s + 3 >= nk ? ra2 : ra1;
    auto mm = [&](int i, int j) __attribute__((always_inline)) {
      if constexpr (FP8) {
        // 32 bytes of k for row i (A) and column j (B): the two 16-byte chunks
        const v8i32 a8 = __builtin_shufflevector(
            __builtin_bit_cast(v4i32_t, av[0][i]), __builtin_bit_cast(v4i32_t, av[1][i]), 0, 1, 2,
            3, 4, 5, 6, 7);
        const v8i32 b8 = __builtin_shufflevector(
            __builtin_bit_cast(v4i32_t, bv[0][j]), __builtin_bit_cast(v4i32_t, bv[1][j]), 0, 1, 2,
            3, 4, 5, 6, 7);
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[i][j], 0, 0, 0, 0,
                                                                     0, 0);
      } else {
        acc[i][j] = mfma32x32x16(av[0][i], bv[0][j], acc[i][j]);
      }
    };
    mm(0, 0);
    if (refill) dma16_asm(rsa, na + (wave * 32) * kRowE, va[0], soff);
    mm(0, 1);
    if (refill) dma16_asm(rsa, na + (wave * 32 + 16) * kRowE, va[1], soff);
    mm(1, 0);
    if (refill) dma16_asm(rw, nb + (wave * 16) * kRowE, vb, soff);
    mm(1, 1);
    if constexpr (!FP8) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(av[1][i], bv[1][j], acc[i][j]);
    }
  };
  for (int s0 = 0; s0 < nst; s0 += 4) {
    stage(s0, sa0, sb0, sa3, sb3);
    if (s0 + 1 < nst) stage(s0 + 1, sa1, sb1, sa0, sb0);
    if (s0 + 2 < nst) stage(s0 + 2, sa2, sb2, sa1, sb1);
    if (s0 + 3 < nst) stage(s0 + 3, sa3, sb3, sa2, sb2);
  }

#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int o = n0 + wn * 64 + j * 32 + l32;
      if (o >= p.h_out) continue;
      const float so = FP8 ? p.sw[o] : 1.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
        if (m >= p.n) continue;
        float v = acc[i][j][r];
        if constexpr (FP8) v = v * p.sx[m] * so;
        if constexpr (F32OUT)
          static_cast<float*>(p.y)[b * p.y_bs + m * p.h_out + o] = v;
        else
          static_cast<uint16_t*>(p.y)[b * p.y_bs + m * p.h_out + o] = f32_to_bf16_bits(v);
      }
    }
  }
}

template <bool F32OUT, bool FP8>
__global__ __launch_bounds__(kNtThreads, 1) void nt_gemm256_kernel(const NtArgs p) {
  nt_tile<F32OUT, FP8>(p, xcd_remap(blockIdx.x, gridDim.x), blockIdx.y);
}

// Several products (instances with their own A, W and Y; shared h_in, h_out)
// in one launch: product g owns the tiles [start[g], start[g + 1]) of the
// XCD-remapped grid.
__global__ __launch_bounds__(kNtThreads, 1) void nt_gemm256_grouped_kernel(const NtGroup grp) {
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  int g = 0;
#pragma unroll 1
  while (g + 1 < grp.n && t >= grp.start[g + 1]) ++g;
  nt_tile<false, false>(grp.p[g], t - grp.start[g], 0);
}

// Buffer-load offsets are 32-bit: the rows of A are run in blocks whose
// bytes stay below 2^31 (each block a launch of its own), and W must fit
// below 2^31 bytes as a whole.
template <bool F32OUT, bool FP8>
hipError_t launch_nt(const NtArgs& a, int batch, hipStream_t stream) {
  constexpr int64_t kEs = FP8 ? 1 : 2;
  const int64_t row_bytes = static_cast<int64_t>(a.h_in) * kEs;
  const int64_t max_rows = (static_cast<int64_t>(INT32_MAX) / row_bytes) / kBM * kBM;
  if (max_rows == 0 || static_cast<int64_t>(a.h_out) * row_bytes > INT32_MAX)
    return hipErrorInvalidValue;
  if (batch == 0) return hipSuccess;
  const int64_t ys = F32OUT ? 4 : 2;
  for (int64_t r0 = 0; r0 < a.n; r0 += max_rows) {
    NtArgs blk = a;
    blk.n = a.n - r0 < max_rows ? a.n - r0 : max_rows;
    blk.a = static_cast<const char*>(a.a) + r0 * row_bytes;
    if (a.a2) blk.a2 = static_cast<const char*>(a.a2) + r0 * row_bytes;
    blk.y = static_cast<char*>(a.y) + r0 * a.h_out * ys;
    if (a.sx) blk.sx = a.sx + r0;
    const int64_t tiles = ((blk.n + kBM - 1) / kBM) * ((a.h_out + kBN - 1) / kBN);
    hipLaunchKernelGGL((nt_gemm256_kernel<F32OUT, FP8>),
                       dim3(static_cast<unsigned>(tiles), batch), dim3(kNtThreads), 0, stream,
                       blk);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

bool nt_gemm256_supported(int h_in) { return h_in > 0 && h_in % kBK == 0; }
bool nt_gemm256_fp8_supported(int h_in) { return h_in > 0 && h_in % 64 == 0; }

hipError_t launch_nt_gemm256_bf16(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t n,
                                  int h_in, int h_out, hipStream_t stream) {
  NtArgs a{x, nullptr, 0, w, 0, y, 0, n, h_in, h_out, nullptr, nullptr};
  return launch_nt<false, false>(a, 1, stream);
}

hipError_t launch_nt_gemm256_fp8(const uint8_t* xq, const float* sx, const uint8_t* wq,
                                 const float* sw, uint16_t* y, int64_t n, int h_in, int h_out,
                                 hipStream_t stream) {
  NtArgs a{xq, nullptr, 0, wq, 0, y, 0, n, h_in, h_out, sx, sw};
  return launch_nt<false, true>(a, 1, stream);
}

hipError_t launch_nt_gemm256_grouped(const NtJob* jobs, int n_jobs, int h_in, int h_out,
                                     hipStream_t stream) {
  if (n_jobs < 1 || n_jobs > kMaxGroup || !nt_gemm256_supported(h_in)) return hipErrorInvalidValue;
  const int64_t row_bytes = static_cast<int64_t>(h_in) * 2;
  if (static_cast<int64_t>(h_out) * row_bytes > INT32_MAX) return hipErrorInvalidValue;
  NtGroup grp{};
  grp.n = n_jobs;
  int64_t total = 0;
  for (int g = 0; g < n_jobs; ++g) {
    const NtJob& j = jobs[g];
    if (j.n < 0 || j.n * row_bytes > INT32_MAX) return hipErrorInvalidValue;
    grp.p[g] = NtArgs{j.x, nullptr, 0, j.w, 0, j.y, 0, j.n, h_in, h_out, nullptr, nullptr};
    grp.start[g] = static_cast<int>(total);
    total += ((j.n + kBM - 1) / kBM) * ((h_out + kBN - 1) / kBN);
    if (total > INT32_MAX) return hipErrorInvalidValue;
  }
  grp.start[n_jobs] = static_cast<int>(total);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(nt_gemm256_grouped_kernel, dim3(static_cast<unsigned>(total)),
                     dim3(kNtThreads), 0, stream, grp);
  return hipGetLastError();
}

hipError_t launch_nt_gemm256_split_f32(const uint16_t* hi, const uint16_t* lo, const uint16_t* w,
                                       float* y, int h, int batch, hipStream_t stream) {
  const int64_t hh = static_cast<int64_t>(h) * h;
  NtArgs a{hi, lo, hh, w, hh, y, hh, static_cast<int64_t>(h), h, h, nullptr, nullptr};
  return launch_nt<true, false>(a, batch, stream);
}

}  // namespace ispa
