// Block-scaled FP8 NT GEMM core for gfx950.
//
// What is computed ("DeepSeek open-source week, day 3: DeepGEMM", "Core
// features" and "Source walk-through" part 3): for every 128-wide K group g,
// an FP8 x FP8 product over that group is formed on the matrix cores, then
// promoted on the vector ALUs into an FP32 accumulator,
//     acc[n][t] += (sa[t][g] * sb[n / 128][g]) * partial_g[n][t],
// and the accumulator is rounded once to BF16 at the end.
//
// gfx950 design (not the page's Hopper design):
//  * One workgroup = 4 waves (one per SIMD) computes a BN x BM tile of D^T:
//    rows are output columns n (the RHS rows), columns are tokens t (the LHS
//    rows).  With the 16x16x128 MFMA, the RHS fragment is src0 and the LHS
//    fragment src1, so each lane ends up holding 4 consecutive n of one
//    token: the token's LHS scale is one per lane and the RHS scale is one
//    per wave (a wave's n range never crosses a 128 block), so promotion
//    costs one multiply per (token, group) and one FMA per output.
//  * One 16x16x128 MFMA spans exactly one scale group, so every partial
//    product is promoted right after its MFMA; no second partial tile of
//    registers is needed.
//  * Operands move HBM -> LDS with the gfx950 direct copy (16 B per lane, no
//    VGPR staging) into STAGES ring slots, each holding one K group of the A
//    tile, the B tile and the tile's BM LHS scales.  Rows are 128 B with a
//    16-byte-chunk XOR swizzle.
//  * Rows beyond the valid range (M/N tails, masked rows past the count) are
//    clamped to the last valid row for loading and are never stored.
#pragma once

#include "device_common.hpp"

namespace fp8g {

enum GemmMode { kDense = 0, kContiguous = 1, kMasked = 2 };

struct GemmParams {
  const uint8_t* a;          // LHS codes
  const float* sa;           // LHS scales, MN-major [KG][sa_ld] (per group for masked)
  const uint8_t* b;          // RHS codes [G][n][k]
  const float* sb;           // RHS scales [G][NB][KG]
  uint16_t* out;             // BF16 output
  float* partial;            // split-K partial sums [splits][m][n] (dense only)
  const int32_t* m_indices;  // contiguous: group of each row
  const int32_t* masked_m;   // masked: valid rows per group
  int64_t sa_ld;
  int m;                     // dense: m; contiguous: m_total; masked: max_m
  int n, k, kg, nb;
  int tiles_m, tiles_n;
  int splits, groups_per_split;
};

// Reads this lane's 32-byte K slice of row `row` of a swizzled [rows][128 B]
// LDS tile: lane l supplies row (l & 15) of a 16-row fragment and K bytes
// [32 * (l >> 4), +32).  The same slice assignment is used for both MFMA
// operands, so the pairing of K elements is consistent.
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int row, int lane) {
  const int c0 = 2 * (lane >> 4);
  const uint8_t* base = tile + row * kRowBytes;
  const v4i x = *reinterpret_cast<const v4i*>(base + 16 * swz(row, c0));
  const v4i y = *reinterpret_cast<const v4i*>(base + 16 * swz(row, c0 + 1));
  v8i r;
  r[0] = x[0]; r[1] = x[1]; r[2] = x[2]; r[3] = x[3];
  r[4] = y[0]; r[5] = y[1]; r[6] = y[2]; r[7] = y[3];
  return r;
}

// Waits until at most `newer` stages of copies issued after the current one
// are still in flight (`copies` per stage per wave), then barriers.
template <int STAGES, int COPIES>
__device__ __forceinline__ void wait_stage(int newer) {
  if constexpr (STAGES >= 3) {
    if (newer >= 1) {
      if constexpr (STAGES >= 4) {
        if (newer >= 2) { wait_vmcnt<2 * COPIES>(); return; }
      }
      wait_vmcnt<COPIES>();
      return;
    }
  }
  wait_vmcnt<0>();
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int MODE, bool SPLIT>
__global__ void __launch_bounds__(256, 1) gemm_kernel(const GemmParams p) {
  static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 16, TN = WN / 16;
  static_assert(WM % 16 == 0 && WN % 16 == 0, "16x16 sub-tiles");
  static_assert(WN <= 128 && 128 % WN == 0, "a wave's n range stays inside one RHS scale block");
  static_assert(BM % 32 == 0 && BN % 32 == 0 && BM <= 256, "whole 8-row copies; scales in one copy");
  static_assert(STAGES >= 2 && STAGES <= 4, "ring depth");
  constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes, S_BYTES = BM * 4;
  constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
  constexpr int A_COPIES = BM / 32, B_COPIES = BN / 32;  // 8-row copies per wave per stage
  static_assert((STAGES - 2) * (A_COPIES + B_COPIES) < 64, "vmcnt range");

  constexpr int SB_BLOCKS = (BN + 127) / 128;  // RHS scale blocks a tile touches
  static_assert(STAGES * STAGE + SB_BLOCKS * kMaxGroups * 4 <= 160 * 1024, "LDS");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE];
  __shared__ float sb_cache[SB_BLOCKS][kMaxGroups];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(threadIdx.x >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // ---- work unit ------------------------------------------------------
  int bid = blockIdx.x;
  int split = 0;
  if constexpr (SPLIT) { split = bid % p.splits; bid /= p.splits; }
  const int n_tile = bid % p.tiles_n;
  bid /= p.tiles_n;
  const int m_tile = bid % p.tiles_m;
  const int group = bid / p.tiles_m;  // masked only
  const int m0 = m_tile * BM, n0 = n_tile * BN;

  const uint8_t* A = p.a;
  const float* SA = p.sa;
  const uint8_t* B = p.b;
  const float* SB = p.sb;
  uint16_t* OUT = p.out;
  int rows = p.m;
  if constexpr (MODE == kContiguous) {
    const int gi = p.m_indices[m0];
    if (gi < 0) return;  // skipped block: output untouched
    B += int64_t(gi) * p.n * p.k;
    SB += int64_t(gi) * p.nb * p.kg;
  } else if constexpr (MODE == kMasked) {
    rows = min(max(p.masked_m[group], 0), p.m);
    if (m0 >= rows) return;  // nothing valid in this tile
    A += int64_t(group) * p.m * p.k;
    SA += int64_t(group) * p.kg * p.sa_ld;
    B += int64_t(group) * p.n * p.k;
    SB += int64_t(group) * p.nb * p.kg;
    OUT += int64_t(group) * p.m * p.n;
  }
  int g_begin = 0, g_end = p.kg;
  if constexpr (SPLIT) {
    g_begin = split * p.groups_per_split;
    g_end = min(p.kg, g_begin + p.groups_per_split);
  }
  const int niter = g_end - g_begin;

  // ---- HBM -> LDS copies of one K group into ring slot `slot` --------------
  const int cp_row = lane >> 3, cp_chunk = lane & 7;
  auto issue = [&](int slot, int g) {
    uint8_t* sA = smem + slot * STAGE;
    uint8_t* sB = sA + A_BYTES;
    uint8_t* sS = sB + B_BYTES;
#pragma unroll
    for (int i = 0; i < A_COPIES; ++i) {
      const int r0 = (i * 4 + wave) * 8;
      const int r = r0 + cp_row;
      const int grow = min(m0 + r, rows - 1);
      copy16_to_lds(A + int64_t(grow) * p.k + g * kGroupK + 16 * swz(r, cp_chunk), sA + r0 * kRowBytes);
    }
#pragma unroll
    for (int i = 0; i < B_COPIES; ++i) {
      const int r0 = (i * 4 + wave) * 8;
      const int r = r0 + cp_row;
      const int grow = min(n0 + r, p.n - 1);
      copy16_to_lds(B + int64_t(grow) * p.k + g * kGroupK + 16 * swz(r, cp_chunk), sB + r0 * kRowBytes);
    }
    if (wave == 0 && lane < BM / 4) {
      const int t = min(m0 + 4 * lane, int(p.sa_ld) - 4);
      copy16_to_lds(SA + int64_t(g) * p.sa_ld + t, sS);
    }
  };

  v4f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int wrow_m = wm * WM, wrow_n = wn * WN;
  // The tile's RHS scale rows go to LDS once, so the K loop reads them
  // without a global load (which would drain the copy queue to be consumed).
#pragma unroll
  for (int b = 0; b < SB_BLOCKS; ++b) {
    const int blk = min(n0 / 128 + b, p.nb - 1);
    for (int g = threadIdx.x; g < p.kg; g += blockDim.x) sb_cache[b][g] = SB[int64_t(blk) * p.kg + g];
  }
  const float* sb_row = sb_cache[wrow_n / 128];
  // sub-tiles of 16 tokens that hold at least one valid token
  const int live_m = min(TM, max(0, (rows - m0 - wrow_m + 15) / 16));

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < niter) issue(s, g_begin + s);

  for (int it = 0; it < niter; ++it) {
    wait_stage<STAGES, A_COPIES + B_COPIES>(min(STAGES - 2, niter - 1 - it));
    wait_lgkmcnt0();
    block_barrier();
    if (it + STAGES - 1 < niter) issue((it + STAGES - 1) % STAGES, g_begin + it + STAGES - 1);

    const int slot = it % STAGES;
    const uint8_t* sA = smem + slot * STAGE;
    const uint8_t* sB = sA + A_BYTES;
    const float* sS = reinterpret_cast<const float*>(sB + B_BYTES);
    const float sbv = sb_row[g_begin + it];

    v8i af[TM];
    float sc[TM];
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      af[j] = read_frag(sA, wrow_m + 16 * j + (lane & 15), lane);
      sc[j] = sS[wrow_m + 16 * j + (lane & 15)] * sbv;
    }
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const v8i bf = read_frag(sB, wrow_n + 16 * i + (lane & 15), lane);
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        if (MODE != kMasked || j < live_m) {
          const v4f pr = mfma16x16x128(bf, af[j]);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(pr[r], sc[j], acc[i][j][r]);
        }
      }
    }
  }

  // ---- epilogue: lane holds n = col..col+3 of one token per sub-tile -------
#pragma unroll
  for (int i = 0; i < TN; ++i) {
    const int col = n0 + wrow_n + 16 * i + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int tok = m0 + wrow_m + 16 * j + (lane & 15);
      if (tok < rows && col < p.n) {
        if constexpr (SPLIT) {
          float* P = p.partial + (int64_t(split) * p.m + tok) * p.n + col;
          *reinterpret_cast<v4f*>(P) = acc[i][j];
        } else {
          uint2 v;
          v.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
          v.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
          *reinterpret_cast<uint2*>(OUT + int64_t(tok) * p.n + col) = v;
        }
      }
    }
  }
}

// Fixed-order sum of split-K partials: out = bf16(p_0 + p_1 + ... + p_{S-1}),
// four outputs per thread.
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* partial, uint16_t* out,
                                                             int64_t mn, int splits) {
  const int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= mn) return;
  v4f s = *reinterpret_cast<const v4f*>(partial + i);
  for (int sp = 1; sp < splits; ++sp) s += *reinterpret_cast<const v4f*>(partial + int64_t(sp) * mn + i);
  uint2 v;
  v.x = pack_bf16x2(s[0], s[1]);
  v.y = pack_bf16x2(s[2], s[3]);
  *reinterpret_cast<uint2*>(out + i) = v;
}

}  // namespace fp8g
