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

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));

// Two FP32 values -> packed BF16 (lo in bits 0..15), rounded to nearest,
// ties to even; a NaN keeps its sign and top payload bits and is made quiet
// ((bits >> 16) | 0x40).  One gfx950 v_cvt_pk_bf16_f32 per pair.  Checked
// on the device against that rounding written out in integer steps
// (u + 0x7fff + ((u >> 16) & 1), then >> 16, with the NaN rule) for every
// FP32 bit pattern in both halves, with FP32 denormals preserved as in these
// kernels: no pattern differs.  (In software the same rounding took about
// nine VALU instructions per value, and converting a 256 x 256 tile took
// about 4.8 us of the large-M kernel's epilogue.)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const v2f v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, v2bf16));
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

// LDS layout of an operand tile of 128-byte rows (one K group of FP8 codes
// per row), in blocks of 16 rows (2 KB).  Row q of a block lives in 256-byte
// line q & 7, half q >> 3, and its logical 16-byte chunk c sits at chunk
// position c ^ (q & 7) of that half:
//     byte(q, c) = 256 * (q & 7) + 128 * (q >> 3) + 16 * (c ^ (q & 7)).
// An MFMA fragment read has lane l fetch row l & 15 at one chunk per 16-lane
// group.  Measured on gfx950, the 16 lanes served together conflict when
// rows 2i and 2i+1 share a 256-byte line (the plain 128-byte-row layout,
// with any XOR swizzle, costs two cycles per read); with rows q and q+8
// paired in a line the reads take one cycle.
__device__ __forceinline__ int tile_byte(int q, int c) {
  return 256 * (q & 7) + 128 * (q >> 3) + 16 * (c ^ (q & 7));
}

// Inverse map used by the copies: the 16-byte slot i (0..63) of half h of a
// 16-row block holds row tile_row(h, i) at logical chunk tile_chunk(h, i).
__device__ __forceinline__ int tile_row(int h, int i) { return 4 * h + (i >> 4) + 8 * ((i >> 3) & 1); }
__device__ __forceinline__ int tile_chunk(int h, int i) { return (i & 7) ^ (tile_row(h, i) & 7); }

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(uintptr_t((const __attribute__((address_space(3))) void*)p));
}

// Uniform (per-wave) value: keeps address arithmetic in scalar registers.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = uint64_t(uintptr_t(p));
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<const void*>(uintptr_t((uint64_t(hi) << 32) | lo));
}

// Direct global -> LDS copy of 16 bytes per lane: lane i's 16 bytes come from
// sbase + voffset (a wave-uniform 64-bit base plus a per-lane 32-bit offset)
// and land at LDS address lds_wave_base + 16 * i (gfx950
// global_load_lds_dwordx4, LDS base in M0).  Issued as inline assembly so
// that the compiler does not track it: the compiler would otherwise wait for
// every outstanding copy before any LDS read it cannot prove disjoint, which
// serialises the prefetch ring.  The callers therefore own the
// synchronisation: wait_vmcnt<N>() retires the copies in issue order, then a
// barrier publishes them to the workgroup.  M0 is written here; these kernels
// use it for nothing else.  Both bases must be the same in every lane (they
// are passed through readfirstlane, which keeps them in scalar registers).
__device__ __forceinline__ void copy16_to_lds(const void* sbase, uint32_t voffset, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(uniform(int(lds_wave_base))), "v"(voffset), "s"(uniform_ptr(sbase)) : "memory");
}

// Same path with 4 bytes per lane (global_load_lds_dword): lane i's dword
// lands at LDS address lds_wave_base + 4 * i.
__device__ __forceinline__ void copy4_to_lds(const void* sbase, uint32_t voffset, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(uniform(int(lds_wave_base))), "v"(voffset), "s"(uniform_ptr(sbase)) : "memory");
}

// Device-coherent 16-byte global store (sc1: past the per-XCD L2s, so
// another XCD sees the data once the store has completed).  Used for split-K
// partial sums that another workgroup, possibly on another XCD, adds up.
__device__ __forceinline__ void store16_coherent(float* p, const v4f& v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" :: "v"(p), "v"(v) : "memory");
}
// S device-coherent 16-byte loads, t[i] = *q[i], issued together and waited
// for (vmcnt(0)) inside one assembly statement: no register of a load still
// in flight is ever visible to the compiler, so it can neither read nor
// reuse one early.  The early-clobber outputs keep every destination apart
// from the addresses of the loads after it.
#define FP8G_LDC(o, i) "global_load_dwordx4 %" #o ", %" #i ", off sc1\n\t"
template <int S>
__device__ __forceinline__ void load16_coherent(const float* const (&q)[S], v4f (&t)[S]) {
  static_assert(S >= 1 && S <= 8, "one to eight loads");
  if constexpr (S == 1) {
    asm volatile(FP8G_LDC(0, 1) "s_waitcnt vmcnt(0)" : "=&v"(t[0]) : "v"(q[0]) : "memory");
  } else if constexpr (S == 2) {
    asm volatile(FP8G_LDC(0, 2) FP8G_LDC(1, 3) "s_waitcnt vmcnt(0)"
                 : "=&v"(t[0]), "=&v"(t[1]) : "v"(q[0]), "v"(q[1]) : "memory");
  } else if constexpr (S == 3) {
    asm volatile(FP8G_LDC(0, 3) FP8G_LDC(1, 4) FP8G_LDC(2, 5) "s_waitcnt vmcnt(0)"
                 : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]) : "v"(q[0]), "v"(q[1]), "v"(q[2]) : "memory");
  } else if constexpr (S == 4) {
    asm volatile(FP8G_LDC(0, 4) FP8G_LDC(1, 5) FP8G_LDC(2, 6) FP8G_LDC(3, 7) "s_waitcnt vmcnt(0)"
                 : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3])
                 : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]) : "memory");
  } else if constexpr (S == 5) {
    asm volatile(FP8G_LDC(0, 5) FP8G_LDC(1, 6) FP8G_LDC(2, 7) FP8G_LDC(3, 8) FP8G_LDC(4, 9) "s_waitcnt vmcnt(0)"
                 : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4])
                 : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(q[4]) : "memory");
  } else if constexpr (S == 6) {
    asm volatile(FP8G_LDC(0, 6) FP8G_LDC(1, 7) FP8G_LDC(2, 8) FP8G_LDC(3, 9) FP8G_LDC(4, 10) FP8G_LDC(5, 11)
                 "s_waitcnt vmcnt(0)"
                 : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5])
                 : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(q[4]), "v"(q[5]) : "memory");
  } else if constexpr (S == 7) {
    asm volatile(FP8G_LDC(0, 7) FP8G_LDC(1, 8) FP8G_LDC(2, 9) FP8G_LDC(3, 10) FP8G_LDC(4, 11) FP8G_LDC(5, 12)
                 FP8G_LDC(6, 13) "s_waitcnt vmcnt(0)"
                 : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6])
                 : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(q[4]), "v"(q[5]), "v"(q[6]) : "memory");
  } else {
    asm volatile(FP8G_LDC(0, 8) FP8G_LDC(1, 9) FP8G_LDC(2, 10) FP8G_LDC(3, 11) FP8G_LDC(4, 12) FP8G_LDC(5, 13)
                 FP8G_LDC(6, 14) FP8G_LDC(7, 15) "s_waitcnt vmcnt(0)"
                 : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]),
                   "=&v"(t[7])
                 : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(q[4]), "v"(q[5]), "v"(q[6]), "v"(q[7])
                 : "memory");
  }
}
#undef FP8G_LDC

// FP8 formats of the operands (the f8f6f4 MFMA's per-operand format codes).
constexpr int kFmtE4M3 = 0, kFmtE5M2 = 1;

// One 16x16x128 FP8 x FP8 -> FP32 MFMA with zero accumulator input.  The
// scaled gfx950 form is used with unit E8M0 scales (127 = 2^0), so it is the
// plain product.  src0 supplies the output rows, src1 the output columns;
// F0 / F1 are their formats (E4M3 or E5M2).
template <int F0 = kFmtE4M3, int F1 = kFmtE4M3>
__device__ __forceinline__ v4f mfma16x16x128(const v8i& src0, const v8i& src1) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(src0, src1, zero, F0, F1, 0, 127, 0, 127);
}

}  // namespace fp8g
