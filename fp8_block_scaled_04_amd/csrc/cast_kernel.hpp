// FP8 casts for gfx950: per-token-group (1 x 128, activations) and per
// 128 x 128 block (weights), to E4M3 (the default) or E5M2.
//
// What is computed (kwkr.cn DeepGEMM usage article, section 3.1 and the code
// in section 4.2; "DeepSeek open-source week, day 3: DeepGEMM", "Basic usage"
// scale shapes): amax = max |x| over the group or block, scale =
// fl32(amax / 448) (1.0 for an all-zero group, a reading the pages leave
// open), q = E4M3(fl32(x / scale)); for E5M2 output 57344 (that format's
// maximum) takes the place of 448.  Division is IEEE fp32 correctly rounded
// (no reciprocal shortcut), so codes and scales are reproducible bit for
// bit.  The hardware conversion rounds to nearest-even; values are first
// clamped to the format's maximum, so the conversion saturates instead of
// producing NaN or infinity past it.
//
// Both kernels are HBM-bound (5 B moved per element, a handful of ALU ops):
// 16-byte loads, one wave-local amax reduction, packed stores.
#pragma once

#include "device_common.hpp"

namespace fp8g {

// Largest finite value of the output format: E4M3 448, E5M2 57344 (the
// "DeepGEMM: FP8 GEMM kernel optimisation practice" page, section 3.1).
template <int FMT>
__device__ __forceinline__ constexpr float fmt_max() { return FMT == kFmtE5M2 ? 57344.0f : 448.0f; }

template <int FMT = kFmtE4M3>
__device__ __forceinline__ float group_scale(float amax) {
  return amax == 0.0f ? 1.0f : __fdiv_rn(amax, fmt_max<FMT>());
}

// Four fp32 -> four codes in one dword (element 0 in the low byte), after a
// clamp to the format's largest finite value (the conversion would give
// NaN or infinity past it).
template <int FMT = kFmtE4M3>
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  constexpr float M = fmt_max<FMT>();
  a = __builtin_amdgcn_fmed3f(a, -M, M);
  b = __builtin_amdgcn_fmed3f(b, -M, M);
  c = __builtin_amdgcn_fmed3f(c, -M, M);
  d = __builtin_amdgcn_fmed3f(d, -M, M);
  int w;
  if constexpr (FMT == kFmtE5M2) {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  }
  return uint32_t(w);
}

__device__ __forceinline__ void load8(const float* x, float v[8]) {
  const float4 a = *reinterpret_cast<const float4*>(x);
  const float4 b = *reinterpret_cast<const float4*>(x + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void load8(const uint16_t* x, float v[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(x);
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Per-token-group cast.  A 1-D grid of ceil(m / 16) * ceil(KG / G)
// workgroups of 256 threads: 16 lanes per (row, group), 8 consecutive
// elements per lane, G consecutive K groups per workgroup with all of their
// loads issued before any is used.  Consecutive workgroups take consecutive
// K groups of the same 16 rows, so the workgroups in flight read long runs
// of each row (a column-stripe order, where they read one 128-element piece
// of many rows, opens a new DRAM page for every piece).  Scales are written
// MN-major, scales[g * ld + row], 16 consecutive rows per workgroup.
template <typename T, int G, int FMT = kFmtE4M3>
__global__ void __launch_bounds__(256) cast_1x128_kernel(const T* __restrict__ x, int m, int k,
                                                         uint8_t* __restrict__ q,
                                                         float* __restrict__ scales, int64_t ld) {
  const unsigned gblocks = (unsigned(k) + kGroupK * G - 1) / (kGroupK * G);
  const int row = int(blockIdx.x / gblocks) * 16 + (threadIdx.x >> 4);
  const int g0 = int(blockIdx.x % gblocks) * G;
  float v[G][8];
#pragma unroll
  for (int u = 0; u < G; ++u) {
    const int col = (g0 + u) * 128 + (threadIdx.x & 15) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[u][i] = 0.f;
    if (row < m && col < k) load8(x + int64_t(row) * k + col, v[u]);
  }
#pragma unroll
  for (int u = 0; u < G; ++u) {
    const int col = (g0 + u) * 128 + (threadIdx.x & 15) * 8;
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[u][i]));
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
    const float s = group_scale<FMT>(amax);
    if (row < m && col < k) {
      uint2 w;
      w.x = fp8x4<FMT>(__fdiv_rn(v[u][0], s), __fdiv_rn(v[u][1], s), __fdiv_rn(v[u][2], s), __fdiv_rn(v[u][3], s));
      w.y = fp8x4<FMT>(__fdiv_rn(v[u][4], s), __fdiv_rn(v[u][5], s), __fdiv_rn(v[u][6], s), __fdiv_rn(v[u][7], s));
      *reinterpret_cast<uint2*>(q + int64_t(row) * k + col) = w;
      if ((threadIdx.x & 15) == 0) scales[int64_t(g0 + u) * ld + row] = s;
    }
  }
}

// 128 x 128 block cast.  A 1-D grid of NB * KG workgroups of 256 threads,
// K blocks fastest (consecutive workgroups read along the same rows).  Each
// load instruction of a wave covers two 512-byte row segments (32 lanes x
// 16 B); a thread holds 16 rows x 4 columns.  k must be a multiple of 4.
template <int FMT = kFmtE4M3>
__global__ void __launch_bounds__(256) cast_128x128_kernel(const float* __restrict__ w, int n, int k,
                                                          uint8_t* __restrict__ q,
                                                          float* __restrict__ scales, int kg) {
  __shared__ float wave_max[4];
  const int nb = int(blockIdx.x / unsigned(kg)), g = int(blockIdx.x % unsigned(kg));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = g * 128 + (lane & 31) * 4;
  const bool col_ok = col < k;
  float4 v[16];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = nb * 128 + wave * 32 + 2 * i + (lane >> 5);
    v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row < n && col_ok) v[i] = *reinterpret_cast<const float4*>(w + int64_t(row) * k + col);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if (lane == 0) wave_max[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
  const float s = group_scale<FMT>(amax);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = nb * 128 + wave * 32 + 2 * i + (lane >> 5);
    if (row < n && col_ok)
      *reinterpret_cast<uint32_t*>(q + int64_t(row) * k + col) =
          fp8x4<FMT>(__fdiv_rn(v[i].x, s), __fdiv_rn(v[i].y, s), __fdiv_rn(v[i].z, s), __fdiv_rn(v[i].w, s));
  }
  if (threadIdx.x == 0) scales[int64_t(nb) * kg + g] = s;
}

}  // namespace fp8g
