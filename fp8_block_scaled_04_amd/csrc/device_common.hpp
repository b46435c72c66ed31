// Device helpers shared by the gfx950 kernels of the block-scaled FP8 GEMM
// library: vector types, BF16 rounding, wait/barrier primitives, the LDS
// swizzle and the direct global->LDS copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8g {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;        // CDNA wavefront
constexpr int kGroupK = 128;     // K width of one scale group (the promotion period)
constexpr int kRowBytes = 128;   // one K group of one FP8 row in LDS
constexpr int kMaxGroups = 512;  // largest K / 128 the GEMM kernels accept (k <= 65536)

// FP32 -> BF16 bits, round to nearest-even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_bits(lo) | (bf16_bits(hi) << 16);
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
}

// Workgroup barrier that is also a compiler barrier for memory operations,
// without the implied wait for every outstanding global load (the pipeline
// waits for exactly the stage it needs with wait_vmcnt before this).
__device__ __forceinline__ void block_barrier() {
  asm volatile("s_barrier" ::: "memory");
}

// LDS swizzle of a [rows][128 B] tile: the 16-byte chunk c of row r is kept
// at chunk position c ^ (r & 7), so the 8 rows read together by one pass of
// a 16-byte-per-lane LDS read land in 8 different chunk columns.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

// Direct global -> LDS copy of 16 bytes per lane: lane i's 16 bytes land at
// lds_wave_base + 16 * i (gfx950 global_load_lds_dwordx4).
__device__ __forceinline__ void copy16_to_lds(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc,
      (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

// Uniform (per-wave) value: keeps address arithmetic in scalar registers.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// One 16x16x128 FP8 x FP8 -> FP32 MFMA with zero accumulator input.  The
// scaled gfx950 form is used with unit E8M0 scales (127 = 2^0), so it is the
// plain product.  src0 supplies the output rows, src1 the output columns.
__device__ __forceinline__ v4f mfma16x16x128(const v8i& src0, const v8i& src1) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(src0, src1, zero, 0, 0, 0, 127, 0, 127);
}

}  // namespace fp8g
