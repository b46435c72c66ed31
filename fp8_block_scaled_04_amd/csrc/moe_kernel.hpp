// MoE layout steps around the grouped GEMMs, for gfx950.
//
// What is computed (the kwkr.cn DeepGEMM usage article, section 3.2 and the
// section 4.3 flow: order the tokens by expert index, count each expert's
// tokens, run the grouped GEMM, put the outputs back in token order; the
// contiguous and masked layouts of "DeepSeek open-source week, day 3:
// DeepGEMM"):
//   counts[g]  = number of tokens routed to expert g;
//   rank[t]    = number of earlier tokens routed to the same expert (the
//                sort is stable, so the layout is unique);
//   contiguous: offsets[g + 1] = offsets[g] + ceil(counts[g] / 128) * 128,
//               dst[t] = offsets[e[t]] + rank[t], m_indices = expert of each
//               row (-1 past the last expert);
//   masked:     dst[t] = e[t] * max_m + rank[t] if rank[t] < max_m else -1,
//               masked_m[g] = min(counts[g], max_m).
// A stable counting sort in three passes: per-chunk histograms, a scan over
// chunks and experts, then ranks within each chunk.  No atomics decide an
// order: LDS atomics only count.
#pragma once

#include "device_common.hpp"

namespace fp8g {

constexpr int kMoeChunk = 1024;      // tokens per workgroup in the counting passes
constexpr int kMoeMaxGroups = 1024;  // experts the layout kernels handle
constexpr int kMoeAlign = 128;       // the contiguous GEMM's row block

__device__ __forceinline__ bool routed(int e, int G) { return e >= 0 && e < G; }

// Pass 1: hist[b][g] = tokens of chunk b routed to g.  Grid: chunks; 256 threads.
__global__ void __launch_bounds__(256) moe_hist_kernel(const int32_t* __restrict__ expert, int T, int G,
                                                       int32_t* __restrict__ hist) {
  __shared__ int cnt[kMoeMaxGroups];
  for (int g = threadIdx.x; g < G; g += blockDim.x) cnt[g] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * kMoeChunk;
  for (int i = threadIdx.x; i < kMoeChunk; i += blockDim.x) {
    const int t = t0 + i;
    if (t < T) {
      const int e = expert[t];
      if (routed(e, G)) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += blockDim.x) hist[int64_t(blockIdx.x) * G + g] = cnt[g];
}

// Pass 2, one workgroup of 1024 threads: replaces hist[b][g] by the tokens
// of g in chunks before b, writes the totals, the aligned offsets
// (contiguous) and the kept counts (masked).
__global__ void __launch_bounds__(1024) moe_scan_kernel(int32_t* __restrict__ hist, int B, int G,
                                                        int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ masked_m, int max_m) {
  __shared__ int part[1024];
  const int g = threadIdx.x;
  int total = 0;
  if (g < G) {
    constexpr int U = 16;  // chunks whose counts are loaded before any is rewritten
    for (int b0 = 0; b0 < B; b0 += U) {
      int c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) c[u] = b0 + u < B ? hist[int64_t(b0 + u) * G + g] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (b0 + u < B) {
          hist[int64_t(b0 + u) * G + g] = total;
          total += c[u];
        }
    }
    counts[g] = total;
    if (masked_m) masked_m[g] = min(total, max_m);
  }
  if (!offsets) return;
  // exclusive scan of the aligned sizes over the experts (Hillis-Steele)
  part[g] = g < G ? (total + kMoeAlign - 1) / kMoeAlign * kMoeAlign : 0;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int v = g >= d ? part[g - d] : 0;
    __syncthreads();
    part[g] += v;
    __syncthreads();
  }
  if (g < G) offsets[g + 1] = part[g];
  if (g == 0) offsets[0] = 0;
}

// Pass 3: destinations.  Grid: chunks; 1024 threads = 16 waves, wave w
// takes tokens [64 w, 64 w + 64) of the chunk.  rank = (tokens of the same
// expert in earlier chunks) + (in earlier waves of this chunk) + (in earlier
// lanes of this wave).
//
// Contiguous layout: the same workgroups also write m_indices[m_rows] (the
// expert whose aligned block range holds each row, -1 past the last one),
// row r by thread r of the grid-wide stride, from the offsets held in LDS.
template <bool CONTIGUOUS>
__global__ void __launch_bounds__(1024) moe_dest_kernel(const int32_t* __restrict__ expert, int T, int G,
                                                        const int32_t* __restrict__ hist,
                                                        const int32_t* __restrict__ offsets, int max_m,
                                                        int32_t* __restrict__ dst, int32_t* __restrict__ m_indices,
                                                        int m_rows) {
  constexpr int NW = kMoeChunk / kWave;
  __shared__ int wave_cnt[NW][kMoeMaxGroups];
  __shared__ int off[CONTIGUOUS ? kMoeMaxGroups + 1 : 1];
  const int t = blockIdx.x * kMoeChunk + threadIdx.x;
  const int e = t < T ? expert[t] : -1;  // in flight while the counts are cleared
  for (int i = threadIdx.x; i < NW * G; i += blockDim.x) wave_cnt[i / G][i % G] = 0;
  if (CONTIGUOUS)
    for (int g = threadIdx.x; g <= G; g += blockDim.x) off[g] = offsets[g];
  __syncthreads();
  if (CONTIGUOUS) {
    for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < m_rows; r += gridDim.x * blockDim.x) {
      int v = -1;
      if (r < off[G]) {
        int lo = 0, hi = G - 1;  // last g with off[g] <= r
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (off[mid] <= r) lo = mid;
          else hi = mid - 1;
        }
        v = lo;
      }
      m_indices[r] = v;
    }
  }
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const bool ok = routed(e, G);
  int in_wave = 0;  // earlier lanes of this wave with the same expert
  if (G <= kWave) {  // one ballot per expert
    const unsigned long long earlier = (1ull << lane) - 1;
    for (int g = 0; g < G; ++g) {
      const unsigned long long m = __ballot(e == g);
      if (e == g) in_wave = __popcll(m & earlier);
    }
  } else {
    for (int j = 0; j < kWave; ++j) {
      const int ej = __shfl(e, j, kWave);
      if (j < lane && ej == e) ++in_wave;
    }
  }
  if (ok) atomicAdd(&wave_cnt[wave][e], 1);
  __syncthreads();
  if (t >= T) return;
  if (!ok) {
    dst[t] = -1;
    return;
  }
  int rank = hist[int64_t(blockIdx.x) * G + e] + in_wave;
  for (int w = 0; w < wave; ++w) rank += wave_cnt[w][e];
  if (CONTIGUOUS) dst[t] = off[e] + rank;
  else dst[t] = rank < max_m ? e * max_m + rank : -1;
}

// Copies `chunks` (> 0) 16-byte pieces with one wave.  Each lane issues 8
// loads before it stores any of them: copied one piece at a time, every
// store would wait for its own load, and a wave would keep only 1 KB in
// flight.  Lanes past the end load the last piece again (unconditional
// loads keep the 8 in flight together) and store nothing.
__device__ __forceinline__ void wave_copy16(const v4i* __restrict__ src, v4i* __restrict__ dst, int chunks,
                                            int lane) {
  constexpr int U = 8;
  for (int c0 = 0; c0 < chunks; c0 += U * kWave) {
    v4i v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[min(c0 + u * kWave + lane, chunks - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave + lane;
      if (c < chunks) dst[c] = v[u];
    }
  }
}

// The one-workgroup layout takes up to 4 x 1024 tokens.  Measured at 8-16
// experts: 5.6-6.0 us against 8.8 us for the three passes at 2048 tokens,
// but 27-28 us against 14.4 us at 16384 tokens (about 1.4 us per round of
// 1024 tokens), so longer routings take the passes.
constexpr int kMoeSmallRounds = 4;

// The whole layout in one workgroup of 1024 threads, for up to
// kMoeSmallRounds * 1024 tokens: the same counting sort as the three passes
// above without their launches.  Thread i takes tokens i, i + 1024, ... (one
// round of 1024 tokens at a time, wave w holding tokens [64 w, 64 w + 64)
// of the round).  Per round:
//   1. each wave counts its tokens per expert: by ballot for up to 64
//      experts (which also gives each token its rank among earlier lanes),
//      else by LDS atomics on the wave's own row of counts;
//   2. 16 lanes per expert (one per wave) turn its counts into exclusive
//      prefixes over the waves by a shuffle scan, starting from the tokens
//      of that expert in earlier rounds;
//   3. rank = that prefix for the token's wave + its rank within the wave.
// Ranks and experts stay in registers until the destinations are written;
// the counts alternate between two buffers, so a round's reads of one never
// meet the next round's writes.  Contiguous: the offsets come from a scan of
// the aligned counts, then the destinations and m_indices[m_rows].  Masked:
// destinations directly, masked_m = min(counts, max_m).
template <bool CONTIGUOUS>
__global__ void __launch_bounds__(1024) moe_layout_small_kernel(const int32_t* __restrict__ expert, int T, int G,
                                                                int max_m, int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ dst,
                                                                int32_t* __restrict__ m_indices, int m_rows,
                                                                int32_t* __restrict__ masked_m) {
  constexpr int NW = 1024 / kWave;
  __shared__ int wave_cnt[2][NW][kMoeMaxGroups];
  __shared__ int base[kMoeMaxGroups + 1];  // tokens per expert so far, then (contiguous) the offsets
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int rounds = (T + 1023) / 1024;
  const bool by_ballot = G <= kWave;
  for (int g = threadIdx.x; g < G; g += blockDim.x) base[g] = 0;
  int e[kMoeSmallRounds], rank[kMoeSmallRounds];
#pragma unroll
  for (int r = 0; r < kMoeSmallRounds; ++r) {  // every load before any use
    const int t = r * 1024 + threadIdx.x;
    e[r] = (r < rounds && t < T) ? expert[t] : -1;
  }
#pragma unroll
  for (int r = 0; r < kMoeSmallRounds; ++r) {
    if (r >= rounds) break;
    int(*cnt)[kMoeMaxGroups] = wave_cnt[r & 1];
    const bool ok = routed(e[r], G);
    int in_wave = 0;  // earlier lanes of this wave with the same expert
    const unsigned long long earlier = (1ull << lane) - 1;
    if (by_ballot) {
      int mine = 0;  // lane g: this wave's tokens of expert g
      for (int g = 0; g < G; ++g) {
        const unsigned long long m = __ballot(e[r] == g);
        if (e[r] == g) in_wave = __popcll(m & earlier);
        if (lane == g) mine = __popcll(m);
      }
      if (lane < G) cnt[wave][lane] = mine;
      __syncthreads();
    } else {
      for (int i = threadIdx.x; i < NW * G; i += blockDim.x) cnt[i / G][i % G] = 0;
      for (int j = 0; j < kWave; ++j) {
        const int ej = __shfl(e[r], j, kWave);
        if (j < lane && ej == e[r]) ++in_wave;
      }
      __syncthreads();
      if (ok) atomicAdd(&cnt[wave][e[r]], 1);
      __syncthreads();
    }
    // 16 consecutive lanes per expert, one per wave: a shuffle scan
    static_assert(NW == 16, "one lane per wave in a 16-lane scan");
    for (int i = threadIdx.x; i < G * NW; i += blockDim.x) {
      const int g = i / NW, w = i % NW;
      const int c = cnt[w][g];
      int v = c;  // inclusive scan over the waves
#pragma unroll
      for (int d = 1; d < NW; d <<= 1) {
        const int u = __shfl_up(v, d, NW);
        if (w >= d) v += u;
      }
      const int b = base[g];
      cnt[w][g] = b + v - c;
      if (w == NW - 1) base[g] = b + v;
    }
    __syncthreads();
    rank[r] = ok ? cnt[wave][e[r]] + in_wave : 0;
  }
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    counts[g] = base[g];
    if (!CONTIGUOUS) masked_m[g] = min(base[g], max_m);
  }
  if constexpr (CONTIGUOUS) {
    // exclusive scan of the aligned sizes over the experts (Hillis-Steele)
    int* part = wave_cnt[0][0];
    const int g = threadIdx.x;
    part[g] = g < G ? (base[g] + kMoeAlign - 1) / kMoeAlign * kMoeAlign : 0;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const int v = g >= d ? part[g - d] : 0;
      __syncthreads();
      part[g] += v;
      __syncthreads();
    }
    if (g < G) base[g + 1] = part[g];  // base[] now holds the offsets
    if (g == 0) base[0] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i <= G; i += blockDim.x) offsets[i] = base[i];
  }
#pragma unroll
  for (int r = 0; r < kMoeSmallRounds; ++r) {
    const int t = r * 1024 + threadIdx.x;
    if (r >= rounds || t >= T) break;
    if (!routed(e[r], G)) dst[t] = -1;
    else if (CONTIGUOUS) dst[t] = base[e[r]] + rank[r];
    else dst[t] = rank[r] < max_m ? e[r] * max_m + rank[r] : -1;
  }
  if constexpr (CONTIGUOUS) {
    for (int row = threadIdx.x; row < m_rows; row += blockDim.x) {
      int v = -1;
      if (row < base[G]) {
        int lo = 0, hi = G - 1;  // last g with base[g] <= row
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (base[mid] <= row) lo = mid;
          else hi = mid - 1;
        }
        v = lo;
      }
      m_indices[row] = v;
    }
  }
}

constexpr int kMoeScaleGroups = 8;  // K groups of scales per thread in the row scatter

// Moves token t's E4M3 row and its KG scales to laid-out row dst[t].
// Workgroups [0, row_blocks) move rows, one wave per token, 16-byte copies
// (k % 16 == 0).  The rest move scales: one thread per token for
// kMoeScaleGroups K groups, 256 consecutive tokens per workgroup, so the
// reads of one K group's scales are coalesced (source MN-major
// [KG][ld_in]) and so are the writes of tokens that land on consecutive
// rows; destination row d lives in group d / rpg at row d % rpg of that
// group's MN-major [KG][ld_out] block.
__global__ void __launch_bounds__(256) moe_scatter_kernel(const uint8_t* __restrict__ q,
                                                          const float* __restrict__ scales, int64_t ld_in,
                                                          int T, int k, const int32_t* __restrict__ dst,
                                                          int rpg, int out_rows, uint8_t* __restrict__ q_out,
                                                          float* __restrict__ scales_out, int64_t ld_out,
                                                          int row_blocks) {
  if (int(blockIdx.x) >= row_blocks) {
    // scale workgroup: 256 tokens x kMoeScaleGroups K groups
    const int kg = (k + 127) / 128;
    const int chunks = (kg + kMoeScaleGroups - 1) / kMoeScaleGroups;
    const int b = blockIdx.x - row_blocks;
    const int t = (b / chunks) * blockDim.x + threadIdx.x;
    const int g0 = (b % chunks) * kMoeScaleGroups;
    if (t >= T) return;
    const int d = dst[t];
    if (d < 0 || d >= out_rows) return;
    float* so = scales_out + int64_t(d / rpg) * kg * ld_out + (d % rpg);
    float v[kMoeScaleGroups];  // all loads in flight before the stores
#pragma unroll
    for (int u = 0; u < kMoeScaleGroups; ++u) v[u] = scales[int64_t(min(g0 + u, kg - 1)) * ld_in + t];
#pragma unroll
    for (int u = 0; u < kMoeScaleGroups; ++u)
      if (g0 + u < kg) so[int64_t(g0 + u) * ld_out] = v[u];
    return;
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6);
  if (t >= T) return;
  const int d = dst[t];
  if (d < 0 || d >= out_rows) return;
  wave_copy16(reinterpret_cast<const v4i*>(q + int64_t(t) * k), reinterpret_cast<v4i*>(q_out + int64_t(d) * k),
              k / 16, lane);
}

// out[t] = y[dst[t]] (BF16 rows, n % 8 == 0), zeros where dst[t] < 0.  One
// wave per token.
__global__ void __launch_bounds__(256) moe_gather_kernel(const uint16_t* __restrict__ y, int n, int y_rows,
                                                         const int32_t* __restrict__ dst, int T,
                                                         uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6);
  if (t >= T) return;
  const int d = dst[t];
  v4i* o = reinterpret_cast<v4i*>(out + int64_t(t) * n);
  if (d < 0 || d >= y_rows) {
    for (int c = lane; c < n / 8; c += kWave) o[c] = v4i{0, 0, 0, 0};
    return;
  }
  wave_copy16(reinterpret_cast<const v4i*>(y + int64_t(d) * n), o, n / 8, lane);
}

}  // namespace fp8g
