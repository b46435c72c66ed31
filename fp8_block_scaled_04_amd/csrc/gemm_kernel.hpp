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

constexpr int kXcds = 8;    // XCDs of an MI355X; workgroups are dealt to them round-robin
constexpr int kGroupM = 4;  // M-tiles walked together in the dense tile order
constexpr int kMaxSplits = 8;  // split-K partials the fix-up adds at most

struct GemmParams {
  const uint8_t* a;          // LHS codes
  const float* sa;           // LHS scales, MN-major [KG][sa_ld] (per group for masked)
  const uint8_t* b;          // RHS codes [G][n][k]
  const float* sb;           // RHS scales [G][NB][KG]
  uint16_t* out;             // BF16 output
  float* partial;            // split-K partial sums [splits][m][n] (dense only)
  unsigned long long* tile_counters;  // split-K arrival counters, one per output tile
  unsigned int tag;          // tag of the split-K arrival counters (never 0)
  const int32_t* m_indices;  // contiguous: group of each row
  const int32_t* masked_m;   // masked: valid rows per group
  int64_t sa_ld;
  int m;                     // dense: m; contiguous: m_total; masked: max_m
  int n, k, kg, nb;
  int tiles_m, tiles_n;
  int splits, groups_per_split;
  int units;                 // work units of the call (tiles, or tiles x splits)
  int unit_offset;           // first unit of this launch (launches under a CU limit take slices)
};

// Loads this lane's 32-byte K slice of one 16-row MFMA fragment from an LDS
// tile laid out by tile_byte().  Lane l supplies row (l & 15) and K bytes
// [32 * (l >> 4), +32), i.e. logical 16-byte chunks c0 = 2 * (l >> 4) and
// c0 + 1; p0 and p1 point at where the layout put those two chunks.  Both
// MFMA operands use the same slice assignment, so K elements pair up
// consistently.
__device__ __forceinline__ v8i lds_frag(const uint8_t* p0, const uint8_t* p1) {
  const v4i x = *reinterpret_cast<const v4i*>(p0);
  const v4i y = *reinterpret_cast<const v4i*>(p1);
  v8i r;
  r[0] = x[0]; r[1] = x[1]; r[2] = x[2]; r[3] = x[3];
  r[4] = y[0]; r[5] = y[1]; r[6] = y[2]; r[7] = y[3];
  return r;
}

// Waits until at most `newer` stages of copies issued after the current one
// are still in flight (`copies` per stage per wave).
template <int STAGES, int COPIES, int N = STAGES - 2>
__device__ __forceinline__ void wait_stage(int newer) {
  if constexpr (N <= 0) {
    wait_vmcnt<0>();
  } else {
    if (newer >= N) { wait_vmcnt<N * COPIES>(); return; }
    wait_stage<STAGES, COPIES, N - 1>(newer);
  }
}

// Promotion of one 16x16 product: acc += scale * partial (one FMA per output).
__device__ __forceinline__ void promote(v4f& acc, const v4f& part, float scale) {
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = fmaf(part[r], scale, acc[r]);
}

// Per-lane LDS pointers of a wave's fragments in ring slot 0: chunk pointers
// for its first 16-row LHS and RHS fragments and its LHS-scale entry.  Later
// fragments sit 16 rows (2048 B) further on, later slots a whole tile on;
// both are compile-time offsets.
struct FragPtrs {
  const uint8_t* a0;
  const uint8_t* a1;
  const uint8_t* b0;
  const uint8_t* b1;
  const float* s;
};

// One K group of a wave's TN x TM sub-tiles, read from ring slot SLOT
// (FMT: bit 0 set = the LHS holds E5M2 codes, bit 1 = the RHS does).  The
// operand with fewer fragments is held in registers, the other is streamed
// one fragment ahead.  Each MFMA is issued before the promotion of the
// previous product, so the promotion FMAs run while the next MFMA occupies
// the matrix core.
// ROW_GUARD (masked layout): only the wave's first live_tm 16-row sub-tiles
// of tokens hold rows below the group's count; the products of the others
// are skipped (their outputs are never stored), so no MFMA or promotion is
// spent on rows past the count.  Each 16-row sub-tile's products are then
// promoted within its own (wave-uniform) branch.
template <int TM, int TN, int A_SLOT, int B_SLOT, int S_SLOT, int FMT = 0, bool ROW_GUARD = false>
__device__ __forceinline__ void group_product(v4f (&acc)[TN][TM], const FragPtrs& f, float sbv, int live_tm = TM) {
  constexpr int FB = (FMT >> 1) & 1, FA = FMT & 1;  // src0 = RHS fragment, src1 = LHS fragment
  constexpr int FRAG = 16 * kRowBytes;
  auto afrag = [&](int j) { return lds_frag(f.a0 + A_SLOT + j * FRAG, f.a1 + A_SLOT + j * FRAG); };
  auto bfrag = [&](int i) { return lds_frag(f.b0 + B_SLOT + i * FRAG, f.b1 + B_SLOT + i * FRAG); };
  auto ascale = [&](int j) { return f.s[S_SLOT / 4 + 16 * j] * sbv; };
  if constexpr (ROW_GUARD) {
    v8i bf[TN];
#pragma unroll
    for (int i = 0; i < TN; ++i) bf[i] = bfrag(i);
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      if (j < live_tm) {
        const v8i a = afrag(j);
        const float sc = ascale(j);
        v4f pr[TN];
#pragma unroll
        for (int i = 0; i < TN; ++i) pr[i] = mfma16x16x128<FB, FA>(bf[i], a);
#pragma unroll
        for (int i = 0; i < TN; ++i) promote(acc[i][j], pr[i], sc);
      }
    }
  } else if constexpr (TN <= TM) {
    v8i bf[TN];
#pragma unroll
    for (int i = 0; i < TN; ++i) bf[i] = bfrag(i);
    v8i a_cur = afrag(0);
    float s_cur = ascale(0);
    v4f prev = {0.f, 0.f, 0.f, 0.f};
    float prev_s = 0.f;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      v8i a_next = a_cur;
      float s_next = s_cur;
      if (j + 1 < TM) {
        a_next = afrag(j + 1);
        s_next = ascale(j + 1);
      }
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const v4f pr = mfma16x16x128<FB, FA>(bf[i], a_cur);
        const int t = j * TN + i;
        if (t > 0) promote(acc[(t - 1) % TN][(t - 1) / TN], prev, prev_s);
        prev = pr;
        prev_s = s_cur;
      }
      a_cur = a_next;
      s_cur = s_next;
    }
    promote(acc[TN - 1][TM - 1], prev, prev_s);
  } else {
    v8i af[TM];
    float sc[TM];
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      af[j] = afrag(j);
      sc[j] = ascale(j);
    }
    v8i b_cur = bfrag(0);
    v4f prev = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      v8i b_next = b_cur;
      if (i + 1 < TN) b_next = bfrag(i + 1);
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const v4f pr = mfma16x16x128<FB, FA>(b_cur, af[j]);
        const int t = i * TM + j;
        if (t > 0) promote(acc[(t - 1) / TM][(t - 1) % TM], prev, sc[(t - 1) % TM]);
        prev = pr;
      }
      b_cur = b_next;
    }
    promote(acc[TN - 1][TM - 1], prev, sc[TM - 1]);
  }
}

template <int N>
struct Int { static constexpr int value = N; };

// Calls f(Int<I>{}) for I = B .. E-1 (compile-time unrolled).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(Int<B>{});
    static_for<B + 1, E>(f);
  }
}

// Tiles of the contiguous layout.  Each aligned 128-row block b carries one
// group index, m_indices[128 b].  A maximal run of blocks with the same
// non-negative index is cut into tiles of two blocks from its first block on
// (the last tile of an odd run has one block), so a 256-row tile never mixes
// two groups and no tile is spent on a group boundary.  Blocks with a
// negative index belong to no tile.  The host cannot know the tile count,
// so every wave derives it from the (L2-resident) index array by a
// wave-wide scan: lane j walks blocks [lo, hi), the j-th chunk of the
// blocks.  The per-lane steps below are plain functions (the host's
// scheduler check runs them too); the wave combines them with shuffles.
struct ContigScan {
  int tiles;  // tiles in total (the same in every lane)
  int lo, hi;
  int in_rs;  // first block of the run in effect just before lo
  int base;   // tiles that start in the chunks of lanes < j
  int count;  // tiles that start in this lane's chunk
};

__host__ __device__ inline int block_group(const int32_t* idx, int b) { return idx[int64_t(b) * 128]; }

// Lane `lane`'s chunk [lo, hi) of the nblk blocks.
__host__ __device__ inline void contig_chunk(int lane, int nblk, int& lo, int& hi) {
  const int chunk = (nblk + kWave - 1) / kWave;
  lo = lane * chunk < nblk ? lane * chunk : nblk;
  hi = lo + chunk < nblk ? lo + chunk : nblk;
}

// First block of the last run that starts in [lo, hi), or -1.
__host__ __device__ inline int contig_last_run_start(const int32_t* idx, int lo, int hi) {
  int last_rs = -1, prev = lo > 0 ? block_group(idx, lo - 1) : 0;
  for (int b = lo; b < hi; ++b) {
    const int e = block_group(idx, b);
    if (b == 0 || e != prev) last_rs = b;
    prev = e;
  }
  return last_rs;
}

// Walks [lo, hi) with in_rs the run start in effect before lo: calls
// f(b) for every block b that starts a tile (an even offset from its run's
// first block, non-negative index) until f returns true; returns the number
// of tile starts visited.
template <typename F>
__host__ __device__ inline int contig_walk(const int32_t* idx, int lo, int hi, int in_rs, F&& f) {
  int cur = in_rs, cnt = 0, prev = lo > 0 ? block_group(idx, lo - 1) : 0;
  for (int b = lo; b < hi; ++b) {
    const int e = block_group(idx, b);
    if (b == 0 || e != prev) cur = b;
    prev = e;
    if (e >= 0 && ((b - cur) & 1) == 0) {
      if (f(b)) break;
      ++cnt;
    }
  }
  return cnt;
}

// Tiles that start in [lo, hi).
__host__ __device__ inline int contig_count(const int32_t* idx, int lo, int hi, int in_rs) {
  return contig_walk(idx, lo, hi, in_rs, [](int) { return false; });
}

// First block of tile t if it starts in this lane's chunk (tiles base ..
// base + count - 1 do), else -1.
__host__ __device__ inline int contig_find(const int32_t* idx, int lo, int hi, int in_rs, int base, int count, int t) {
  if (t < base || t >= base + count) return -1;
  int found = -1, k = base;
  contig_walk(idx, lo, hi, in_rs, [&](int b) {
    if (k == t) { found = b; return true; }
    ++k;
    return false;
  });
  return found;
}

// Blocks (1 or 2) of the tile that starts at `block`.
__host__ __device__ inline int contig_tile_blocks(const int32_t* idx, int nblk, int block) {
  return (block + 1 < nblk && block_group(idx, block + 1) == block_group(idx, block)) ? 2 : 1;
}

__device__ __forceinline__ ContigScan contiguous_scan(const int32_t* idx, int nblk) {
  const int lane = threadIdx.x & (kWave - 1);
  ContigScan s;
  contig_chunk(lane, nblk, s.lo, s.hi);
  int v = contig_last_run_start(idx, s.lo, s.hi);  // inclusive max-scan over lanes
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int t = __shfl_up(v, d, kWave);
    if (lane >= d) v = max(v, t);
  }
  const int excl = __shfl_up(v, 1, kWave);
  s.in_rs = lane == 0 ? -1 : excl;
  const int cnt = contig_count(idx, s.lo, s.hi, s.in_rs);
  s.count = cnt;
  int incl = cnt;  // inclusive sum-scan over lanes
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int t = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += t;
  }
  s.base = incl - cnt;
  s.tiles = uniform(__shfl(incl, kWave - 1, kWave));
  return s;
}

// First block, block count (1 or 2) and group of tile t (0 <= t < tiles).
__device__ __forceinline__ void contiguous_locate(const ContigScan& s, const int32_t* idx, int nblk, int t,
                                                  int& block, int& nblocks, int& group) {
  const int found = contig_find(idx, s.lo, s.hi, s.in_rs, s.base, s.count, t);
  const unsigned long long who = __ballot(found >= 0);
  block = uniform(__shfl(found, __ffsll(who) - 1, kWave));
  group = uniform(block_group(idx, block));
  nblocks = uniform(contig_tile_blocks(idx, nblk, block));
}

// Logical unit of workgroup `bid` when `total` units are dealt to the XCDs:
// workgroups reach the 8 XCDs round-robin (bid % 8) and each XCD has its
// own L2, so XCD x takes the x-th contiguous share of the logical order
// (shares differ by at most one unit).  -1 when this workgroup's slot is
// past its XCD's share.  A bijection from the workgroups with a unit onto
// [0, total), so correctness does not depend on the dispatch order.
__host__ __device__ inline int xcd_logical(int bid, int total) {
  const int xcd = bid % kXcds, slot = bid / kXcds;
  const int per = total / kXcds, extra = total % kXcds;
  if (slot >= per + (xcd < extra ? 1 : 0)) return -1;
  return (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) + slot;
}

// Dense (and contiguous) tile of logical unit L: the split fastest, then
// bands of kGroupM M-tiles by all N-tiles, M fastest within a band, so the
// tiles an XCD runs at once share a few A and B K-slices.
__host__ __device__ inline void dense_tile(int L, int tiles_m, int tiles_n, int splits, int& m_tile, int& n_tile,
                                           int& split) {
  split = L % splits;
  L /= splits;
  const int band = kGroupM * tiles_n;
  const int first_m = (L / band) * kGroupM;
  const int rows_in_band = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
  const int in_band = L % band;
  m_tile = first_m + in_band % rows_in_band;
  n_tile = in_band / rows_in_band;
}

// Work units of the masked layout.  Group g has ceil(rows_g / BM) live row
// tiles (rows_g = masked_m[g] clamped to [0, max_m]) for each of the tiles_n
// column tiles; only these units have work.  They are numbered group by
// group, column tile by column tile, row tile fastest, and XCD x takes the
// x-th contiguous eighth of that numbering.  So the row tiles that share an
// RHS tile run together on one XCD (the tile reaches that XCD's L2 once), a
// group's LHS rows are fetched by the one or two XCDs its units fall on
// (not by all eight), and every XCD gets the same number of live units.
// Every wave derives the numbering from the (L2-resident) counts.  Returns
// false for a workgroup past the live units of its XCD.
__host__ __device__ inline int masked_live_tiles(int count, int max_m, int bm) {
  const int rows = count < 0 ? 0 : (count > max_m ? max_m : count);
  return (rows + bm - 1) / bm;
}

template <int BM>
__device__ __forceinline__ bool masked_unit(const int32_t* masked_m, int groups, int max_m, int tiles_n, int bid,
                                            int& group, int& m_tile, int& n_tile) {
  const int lane = threadIdx.x & (kWave - 1);
  auto live_tiles = [&](int g) { return g < groups ? masked_live_tiles(masked_m[g], max_m, BM) : 0; };
  auto inclusive_sum = [&](int v) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int t = __shfl_up(v, d, kWave);
      if (lane >= d) v += t;
    }
    return v;
  };
  int total = 0;  // live units (< the grid size, so no overflow)
  for (int g0 = 0; g0 < groups; g0 += kWave)
    total += uniform(__shfl(inclusive_sum(live_tiles(g0 + lane) * tiles_n), kWave - 1, kWave));
  const int L = xcd_logical(bid, total);
  if (L < 0) return false;
  int base = 0;
  for (int g0 = 0; g0 < groups; g0 += kWave) {
    const int mt = live_tiles(g0 + lane);
    const int u = mt * tiles_n;
    const int incl = inclusive_sum(u);
    const int first = base + incl - u;  // this lane's group's first unit
    const unsigned long long who = __ballot(u > 0 && L >= first && L < first + u);
    if (who) {
      const int src = __ffsll(who) - 1;
      const int mtg = uniform(__shfl(mt, src, kWave));
      const int r = L - uniform(__shfl(first, src, kWave));
      group = g0 + src;
      m_tile = r % mtg;
      n_tile = r / mtg;
      return true;
    }
    base += uniform(__shfl(incl, kWave - 1, kWave));
  }
  return false;  // not reached: L < total
}

// ---- epilogue ---------------------------------------------------------------
// Writes a workgroup's BM x BN tile from the accumulators of the waves that
// hold it (holder): wave (wrow_m, wrow_n) holds tokens wrow_m.. and outputs
// wrow_n.. of the tile as acc[i][j] = sub-tile (n 16 i.., token 16 j..), each
// lane 4 consecutive n of one token.  smem (at least epilogue_lds<BM, BN>(SPLIT)
// bytes, free once the K loop is done) stages the tile.  Every thread of the
// workgroup calls it.
template <int BM, int BN>
constexpr int epilogue_lds(bool split) {
  return split ? BM * (BN + 4) * 4 : BM * (BN + 8) * 2;
}

template <int BM, int BN, int TM, int TN, bool SPLIT>
__device__ __forceinline__ void write_tile(const GemmParams& p, const v4f (&acc)[TN][TM], uint8_t* smem, bool holder,
                                           int wrow_m, int wrow_n, int m0, int n0, int rows, int shape_n, int split,
                                           int m_tile, int n_tile, uint16_t* OUT) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int OUT_LDT = BN + 8;  // padded row stride (elements) of the staged BF16 tile
  if constexpr (SPLIT) {
    // Publish this split's partial tile, then count arrivals on the tile.
    // The last workgroup to arrive adds all partials in split order
    // (p_0 + p_1 + ... + p_{S-1}), so the result does not depend on arrival
    // order.  The tile is staged through LDS (free once the K loop is done)
    // so that partials move as whole rows of 16-byte device-coherent
    // accesses, which go past the per-XCD L2s: retiring the stores before
    // the arrival is counted makes them visible to the last workgroup
    // without any cache-wide write-back or invalidate.
    constexpr int LDT = BN + 4;  // padded row stride (floats) of the staged tile
    constexpr int CHUNKS = BM * BN / 4;
    float* stage = reinterpret_cast<float*>(smem);
    __syncthreads();  // every wave is done with the ring (and with the partial-tile sums)
    if (holder) {
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
          *reinterpret_cast<v4f*>(stage + (wrow_m + 16 * j + (lane & 15)) * LDT + wrow_n + 16 * i + 4 * (lane >> 4)) =
              acc[i][j];
    }
    __syncthreads();
    const int64_t mn = int64_t(p.m) * shape_n;
    for (int c = threadIdx.x; c < CHUNKS; c += blockDim.x) {
      const int r = c / (BN / 4), c4 = 4 * (c % (BN / 4));
      if (m0 + r < rows && n0 + c4 < shape_n)
        store16_coherent(p.partial + split * mn + int64_t(m0 + r) * shape_n + n0 + c4,
                         *reinterpret_cast<const v4f*>(stage + r * LDT + c4));
    }
    __shared__ int last_arrival;
    // counter word: tag in the high 32 bits, arrivals in the low 32.  The
    // last arrival leaves the word at (tag, 0), so a word carrying this
    // call's tag counts arrivals from zero, and nothing but this call's
    // arrivals touches it (calls sharing a workspace run one after
    // another): a fetch-and-add counts the arrival in one round trip.  A
    // word with another tag (uninitialised memory, partial sums of another
    // configuration, a counter left by a launch that failed part-way) is
    // replaced by (tag, 1) with a compare-and-swap, which, if some other
    // arrival got there first, returns the word as it now is.  The word is
    // fetched while the partial's stores are still in flight; the arrival
    // itself is counted after every store has completed.
    unsigned long long* ctr = p.tile_counters + (int64_t(m_tile) * p.tiles_n + n_tile);
    unsigned long long seen = 0;
    if (threadIdx.x == 0) seen = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_vmcnt<0>();
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long old = seen;
      unsigned long long nxt;
      for (;;) {
        if (unsigned(old >> 32) == p.tag) {
          nxt = __hip_atomic_fetch_add(ctr, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
          break;
        }
        nxt = ((unsigned long long)p.tag << 32) | 1ull;
        if (__hip_atomic_compare_exchange_strong(ctr, &old, nxt, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT))
          break;
      }
      const bool last = unsigned(nxt) == unsigned(p.splits);
      if (last) __hip_atomic_store(ctr, (unsigned long long)p.tag << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_arrival = last;
    }
    __syncthreads();
    if (!last_arrival) return;
    // Every split's partial of a 4-wide chunk (this one's too, read back
    // like the others) is requested before one wait, then added in split
    // order.  With few splits a thread takes several chunks per wait (at
    // most eight loads in flight), so a tile of more chunks than threads
    // costs one or two memory round trips instead of one per chunk.  A
    // chunk past the tile's edge reads the nearest chunk inside it and
    // writes nothing.
    auto add_partials = [&](auto s_tag) {
      constexpr int S = decltype(s_tag)::value;
      constexpr int G = 8 / S;
      for (int c0 = threadIdx.x; c0 < CHUNKS; c0 += G * blockDim.x) {
        const float* q[G * S];
        int64_t at[G];
        bool live[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int c = c0 + g * blockDim.x;
          const int r = c / (BN / 4), c4 = 4 * (c % (BN / 4));
          live[g] = c < CHUNKS && m0 + r < rows && n0 + c4 < shape_n;
          // clamped into the tile (a live chunk keeps its place); written
          // without a select against the tile's base so that the tile
          // indices stay in scalar registers for the whole kernel
          const int rr = min(r, min(BM, rows - m0) - 1), cc = min(c4, min(BN, shape_n - n0) - 4);
          at[g] = int64_t(m0 + rr) * shape_n + n0 + cc;
#pragma unroll
          for (int sp = 0; sp < S; ++sp) q[g * S + sp] = p.partial + at[g] + sp * mn;
        }
        v4f t[G * S];
        load16_coherent<G * S>(q, t);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          if (!live[g]) continue;
          v4f sum = t[g * S];
#pragma unroll
          for (int sp = 1; sp < S; ++sp) sum += t[g * S + sp];
          uint2 v;
          v.x = pack_bf16x2(sum[0], sum[1]);
          v.y = pack_bf16x2(sum[2], sum[3]);
          *reinterpret_cast<uint2*>(OUT + at[g]) = v;
        }
      }
    };
    static_assert(kMaxSplits == 8, "one case per split count");
    switch (p.splits) {
      case 1: add_partials(Int<1>{}); break;
      case 2: add_partials(Int<2>{}); break;
      case 3: add_partials(Int<3>{}); break;
      case 4: add_partials(Int<4>{}); break;
      case 5: add_partials(Int<5>{}); break;
      case 6: add_partials(Int<6>{}); break;
      case 7: add_partials(Int<7>{}); break;
      default: add_partials(Int<8>{}); break;
    }
  } else {
    // The tile goes out through LDS: a lane's accumulators are 4 columns of
    // one row per sub-tile, so stored directly each instruction would write
    // 32 bytes into each of 16 rows; staged, every instruction writes whole
    // rows in 16-byte pieces (measured: the output burst at the end of a
    // round of large-M tiles drains about twice as fast).
    uint16_t* stage = reinterpret_cast<uint16_t*>(smem);
    __syncthreads();  // every wave is done with the ring (and with the partial-tile sums)
    if (holder) {
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) {
          uint2 v;
          v.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
          v.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
          *reinterpret_cast<uint2*>(stage + (wrow_m + 16 * j + (lane & 15)) * OUT_LDT + wrow_n + 16 * i +
                                    4 * (lane >> 4)) = v;
        }
    }
    __syncthreads();
    constexpr int CHUNKS = BN / 8;  // 16-byte pieces per tile row (n % 8 == 0: a piece is all in or all out)
    for (int c = threadIdx.x; c < BM * CHUNKS; c += blockDim.x) {
      const int r = c / CHUNKS, col = n0 + 8 * (c % CHUNKS);
      if (m0 + r < rows && col < shape_n)
        *reinterpret_cast<uint4*>(OUT + int64_t(m0 + r) * shape_n + col) =
            *reinterpret_cast<const uint4*>(stage + r * OUT_LDT + 8 * (c % CHUNKS));
    }
  }
}

// KU consecutive K groups share one ring stage (one wait and one barrier),
// and WK waves (dividing KU) may share each sub-tile, taking every WK-th
// group of a stage; their partial tiles are added in LDS, in wave order,
// after the K loop.  With few tokens a group's products are too short to
// cover the fixed latency of a stage's synchronisation and LDS reads; giving
// each wave its own groups of a larger sub-tile keeps several independent
// chains of MFMAs in flight.
// FMT selects the operand formats (bit 0: LHS E5M2, bit 1: RHS E5M2).
// NSPEC / KSPEC > 0 make n / k compile-time constants (the runtime
// specialisation builds them per shape); 0 takes them from the parameters.
template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int MODE, bool SPLIT, int KU = 1, int WK = 1,
          int FMT = 0, int NSPEC = 0, int KSPEC = 0>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N * WK, 1) gemm_kernel(const GemmParams p) {
  constexpr int NW = WAVES_M * WAVES_N * WK;  // 4 waves: one per SIMD; 8 waves: two per SIMD
  static_assert(NW == 4 || NW == 8, "four or eight waves per workgroup");
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 16, TN = WN / 16;
  static_assert(WM % 16 == 0 && WN % 16 == 0, "16x16 sub-tiles");
  static_assert(WN <= 128 && 128 % WN == 0, "a wave's n range stays inside one RHS scale block");
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0 && BM <= 256, "whole 1 KB copies; scales in one copy");
  // STAGES == 1 is the single-buffer debug form: each stage's copies are
  // issued only after every wave has finished reading the previous one, so
  // loads never overlap the products ("DeepGEMM: FP8 GEMM kernel
  // optimisation practice on Hopper Tensor Cores", section 6.2: fall back
  // to one buffer to tell a pipeline race from an arithmetic error).
  static_assert(STAGES >= 1 && STAGES <= 8 && KU >= 1 && KU <= 4 && KU % WK == 0, "ring depth");
  // LDS: [STAGES * KU][BM][128 B] LHS tiles, then [STAGES * KU][BN][128 B]
  // RHS tiles, then [STAGES * KU][BM] LHS scales (one group per slot, KU
  // slots per stage), then the tile's RHS scale rows.
  constexpr int SLOTS = STAGES * KU;
  constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes, S_BYTES = BM * 4;
  constexpr int A_REGION = 0, B_REGION = SLOTS * A_BYTES, S_REGION = B_REGION + SLOTS * B_BYTES;
  constexpr int RING = S_REGION + SLOTS * S_BYTES;
  constexpr int A_COPIES = BM / (8 * NW), B_COPIES = BN / (8 * NW);  // 8-row copies per wave per group
  constexpr int STAGE_COPIES = KU * (A_COPIES + B_COPIES);
  static_assert((STAGES - 2) * STAGE_COPIES < 64, "vmcnt range");
  constexpr int SB_BLOCKS = (BN + 127) / 128;  // RHS scale blocks a tile touches
  static_assert(RING + SB_BLOCKS * kMaxGroups * 4 <= 160 * 1024, "LDS");

  // After the K loop the ring holds the BF16 output tile on its way out
  // (rows padded by 8 elements so that neither the fragment-ordered writes
  // nor the row-ordered reads pile onto a few banks).
  // A split's FP32 partial tile is staged the same way (rows padded by 4).
  constexpr int EPI = epilogue_lds<BM, BN>(SPLIT);
  constexpr int SMEM = RING > EPI ? RING : EPI;
  static_assert(SMEM + SB_BLOCKS * kMaxGroups * 4 <= 160 * 1024, "LDS with the output staging");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];
  __shared__ float sb_cache[SB_BLOCKS][kMaxGroups];

  static_assert(NSPEC >= 0 && NSPEC % 8 == 0 && KSPEC >= 0 && KSPEC % kGroupK == 0 &&
                KSPEC <= kGroupK * kMaxGroups, "specialised shape");
  const int shape_n = NSPEC > 0 ? NSPEC : p.n;
  const int shape_k = KSPEC > 0 ? KSPEC : p.k;
  const int shape_kg = KSPEC > 0 ? KSPEC / kGroupK : p.kg;
  const int shape_nb = NSPEC > 0 ? (NSPEC + 127) / 128 : p.nb;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(threadIdx.x >> 6);
  const int wk = wave / (WAVES_M * WAVES_N);  // which groups of a stage this wave multiplies
  const int wm = (wave % (WAVES_M * WAVES_N)) / WAVES_N, wn = wave % WAVES_N;

  // ---- work unit ------------------------------------------------------
  // Unit blockIdx.x + p.unit_offset of p.units: a launch covers all units,
  // or, under a CU limit, one of several consecutive slices of them.
  [[maybe_unused]] const int bid = blockIdx.x + p.unit_offset;
  int split = 0;
  int n_tile, m_tile, group = 0;
  int tiles_m = p.tiles_m;
  [[maybe_unused]] ContigScan cs;
  if constexpr (MODE == kContiguous) {
    // p.units is the largest possible tile count; units past the real count
    // have nothing to do
    cs = contiguous_scan(p.m_indices, p.m / 128);
    tiles_m = cs.tiles;
    if (bid >= tiles_m * p.tiles_n) return;
  }
  if constexpr (MODE == kDense) {
    // Each launch deals its own units [unit_offset, unit_offset + gridDim.x)
    // to the XCDs (all of them when there is no CU limit), so that every
    // slice of a CU-limited call also keeps the tiles that run together on
    // one XCD; every workgroup of the launch has a unit.
    const int L = p.unit_offset + xcd_logical(blockIdx.x, gridDim.x);
    dense_tile(L, tiles_m, p.tiles_n, SPLIT ? p.splits : 1, m_tile, n_tile, split);
  } else if constexpr (MODE == kContiguous) {
    // (every workgroup below the tile count has a unit: bid < total)
    const int L = xcd_logical(bid, tiles_m * p.tiles_n);
    dense_tile(L, tiles_m, p.tiles_n, 1, m_tile, n_tile, split);
  } else {
    // (p.units counts every possible unit: groups x tiles_m x tiles_n)
    if (!masked_unit<BM>(p.masked_m, p.units / (p.tiles_m * p.tiles_n), p.m, p.tiles_n, bid, group,
                         m_tile, n_tile))
      return;
  }
  int m0 = m_tile * BM;
  const int n0 = n_tile * BN;

  const uint8_t* A = p.a;
  const float* SA = p.sa;
  const uint8_t* B = p.b;
  const float* SB = p.sb;
  uint16_t* OUT = p.out;
  int rows = p.m;
  if constexpr (MODE == kContiguous) {
    static_assert(BM == 256, "contiguous tiles are one or two 128-row blocks");
    int block, nblocks, gi;
    contiguous_locate(cs, p.m_indices, p.m / 128, m_tile, block, nblocks, gi);
    m0 = 128 * block;
    rows = m0 + 128 * nblocks;  // rows of other blocks are neither used nor written
    B += int64_t(gi) * shape_n * shape_k;
    SB += int64_t(gi) * shape_nb * shape_kg;
  } else if constexpr (MODE == kMasked) {
    rows = min(max(p.masked_m[group], 0), p.m);
    if (m0 >= rows) return;  // nothing valid in this tile
    A += int64_t(group) * p.m * shape_k;
    SA += int64_t(group) * shape_kg * p.sa_ld;
    B += int64_t(group) * shape_n * shape_k;
    SB += int64_t(group) * shape_nb * shape_kg;
    OUT += int64_t(group) * p.m * shape_n;
  }
  int g_begin = 0, g_end = shape_kg;
  if constexpr (SPLIT) {
    g_begin = split * p.groups_per_split;
    g_end = min(shape_kg, g_begin + p.groups_per_split);
  }
  const int ngroups = g_end - g_begin;
  const int niter = (ngroups + KU - 1) / KU;  // ring stages

  // ---- HBM -> LDS copies: per-lane byte offsets are loop invariant --------
  // Copy i of this wave fills 1 KB unit u = i * NW + wave of the tile, i.e.
  // half u & 1 of 16-row block u >> 1: lane l fetches the row and logical
  // chunk that tile_byte() places at byte 16 * l of that unit.  The 64-bit
  // bases point at the tile's first row (and scale), so the 32-bit per-lane
  // offsets stay below BM (or BN) rows of k bytes however large the operands
  // are (an operand past 4 GiB would overflow offsets taken from its start).
  const uint8_t* A_tile = A + int64_t(m0) * shape_k;
  const uint8_t* B_tile = B + int64_t(n0) * shape_k;
  const float* SA_tile = SA + m0;
  uint32_t a_off[A_COPIES], b_off[B_COPIES];
#pragma unroll
  for (int i = 0; i < A_COPIES; ++i) {
    const int u = i * NW + wave;
    const int r = 16 * (u >> 1) + tile_row(u & 1, lane);
    a_off[i] = uint32_t(min(m0 + r, rows - 1) - m0) * uint32_t(shape_k) + 16u * tile_chunk(u & 1, lane);
  }
#pragma unroll
  for (int i = 0; i < B_COPIES; ++i) {
    const int u = i * NW + wave;
    const int r = 16 * (u >> 1) + tile_row(u & 1, lane);
    b_off[i] = uint32_t(min(n0 + r, shape_n - 1) - n0) * uint32_t(shape_k) + 16u * tile_chunk(u & 1, lane);
  }
  // (sa_ld >= rows and a multiple of 4, and m0 a multiple of 4 below rows:
  // the clamped index is never below m0)
  const uint32_t s_off = 4u * uint32_t(min(m0 + 4 * lane, int(p.sa_ld) - 4) - m0);
  const uint32_t lds0 = uniform(int(lds_addr(smem)));
  // Stage `it` holds groups g_begin + KU * it + u, u < KU; in a last,
  // partial stage the missing groups repeat the last one (never multiplied),
  // so every stage issues the same number of copies.
  auto issue = [&](auto stage_tag, int it) {
    constexpr int stage = decltype(stage_tag)::value;
    static_for<0, KU>([&](auto uc) __attribute__((always_inline)) {
      constexpr int slot = stage * KU + decltype(uc)::value;
      const int g = uniform(min(g_begin + KU * it + decltype(uc)::value, g_end - 1));
      const uint8_t* a_src = A_tile + int64_t(g) * kGroupK;
      const uint8_t* b_src = B_tile + int64_t(g) * kGroupK;
#pragma unroll
      for (int i = 0; i < A_COPIES; ++i)
        copy16_to_lds(a_src, a_off[i], lds0 + A_REGION + slot * A_BYTES + (i * NW + wave) * 1024);
#pragma unroll
      for (int i = 0; i < B_COPIES; ++i)
        copy16_to_lds(b_src, b_off[i], lds0 + B_REGION + slot * B_BYTES + (i * NW + wave) * 1024);
      if (wave == 0 && lane < BM / 4)
        copy16_to_lds(SA_tile + int64_t(g) * p.sa_ld, s_off, lds0 + S_REGION + slot * S_BYTES);
    });
  };

  v4f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int wrow_m = wm * WM, wrow_n = wn * WN;
  // The tile's RHS scale rows (this split's K groups) go to LDS once, by the
  // same direct copy and ahead of the operand copies, so the first ring wait
  // also covers them and the K loop reads them without a global load.
  {
    const uint32_t sb_lds = uniform(int(lds_addr(&sb_cache[0][0])));
    for (int c = wave; c < SB_BLOCKS * ((ngroups + 63) / 64); c += NW) {
      const int b = c % SB_BLOCKS, part = c / SB_BLOCKS;
      const int blk = min(n0 / 128 + b, shape_nb - 1);
      const int g = min(g_begin + 64 * part + lane, g_end - 1);
      copy4_to_lds(SB + int64_t(blk) * shape_kg, 4u * uint32_t(g), sb_lds + 4 * (b * kMaxGroups + 64 * part));
    }
  }
  const float* sb_row = sb_cache[wrow_n / 128];
  // A wave whose tokens are all past the tile's valid rows (masked counts,
  // one-block contiguous tiles) skips the products (its copies still run:
  // the ring is shared); in the masked layout a live wave also skips its
  // 16-row sub-tiles that lie wholly past the count.
  const bool wave_live = MODE == kDense || m0 + wrow_m < rows;
  const int live_tm = MODE == kMasked ? uniform(min(TM, max(0, (rows - m0 - wrow_m + 15) / 16))) : TM;

  // Fragment pointers of ring slot wk (wave and fragment row offsets are
  // multiples of 16, i.e. whole 2 KB blocks).
  const int lr = lane & 15, c0 = 2 * (lane >> 4);
  FragPtrs f;
  f.a0 = smem + A_REGION + wk * A_BYTES + wrow_m * kRowBytes + tile_byte(lr, c0);
  f.a1 = smem + A_REGION + wk * A_BYTES + wrow_m * kRowBytes + tile_byte(lr, c0 + 1);
  f.b0 = smem + B_REGION + wk * B_BYTES + wrow_n * kRowBytes + tile_byte(lr, c0);
  f.b1 = smem + B_REGION + wk * B_BYTES + wrow_n * kRowBytes + tile_byte(lr, c0 + 1);
  f.s = reinterpret_cast<const float*>(smem + S_REGION + wk * S_BYTES) + wrow_m + lr;

  // (the scale-row copies above are older)
  static_for<0, (STAGES > 1 ? STAGES - 1 : 1)>([&](auto ic) __attribute__((always_inline)) {
    constexpr int I = decltype(ic)::value;
    if (I < niter) issue(Int<I>{}, I);
  });

  auto step = [&](auto stage_tag, int it) {
    constexpr int stage = decltype(stage_tag)::value;
    wait_stage<STAGES, STAGE_COPIES>(min(STAGES - 2, niter - 1 - it));
    wait_lgkmcnt0();
    block_barrier();
    if constexpr (STAGES > 1)
      if (it + STAGES - 1 < niter) issue(Int<(stage + STAGES - 1) % STAGES>{}, it + STAGES - 1);
    if (wave_live)
      static_for<0, KU / WK>([&](auto uc) __attribute__((always_inline)) {
        constexpr int slot = stage * KU + decltype(uc)::value * WK;  // + wk, folded into f
        const int gl = KU * it + decltype(uc)::value * WK + wk;
        if (KU == 1 || gl < ngroups)
          group_product<TM, TN, slot * A_BYTES, slot * B_BYTES, slot * S_BYTES, FMT, MODE == kMasked>(
              acc, f, sb_row[gl], live_tm);
      });
    if constexpr (STAGES == 1) {
      // every wave's reads of the only slot are done before it is refilled
      wait_lgkmcnt0();
      block_barrier();
      if (it + 1 < niter) issue(Int<0>{}, it + 1);
    }
  };
  // Kept rolled: with k a compile-time constant the compiler would unroll
  // the whole K loop, run out of registers and spill, and spill traffic
  // would share the vector-memory counter the ring waits count copies with.
#pragma clang loop unroll(disable)
  for (int it = 0; it < niter; it += STAGES) {
    static_for<0, STAGES>([&](auto ic) __attribute__((always_inline)) {
      constexpr int I = decltype(ic)::value;
      if (it + I < niter) step(Int<I>{}, it + I);
    });
  }

  // ---- waves sharing a sub-tile add their partial tiles (wave order) ------
  if constexpr (WK > 1) {
    constexpr int PART = TN * TM * kWave;  // v4f elements of one wave's sub-tile
    static_assert(NW * PART * 16 <= RING, "partial tiles fit in the ring");
    v4f* red = reinterpret_cast<v4f*>(smem);
    __syncthreads();  // every wave is done with the ring
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) red[(wave * TN + i) * TM * kWave + j * kWave + lane] = acc[i][j];
    __syncthreads();
    if (wk == 0) {
#pragma unroll
      for (int w = 1; w < WK; ++w) {
        const int other = w * WAVES_M * WAVES_N + wave;
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int j = 0; j < TM; ++j) acc[i][j] += red[(other * TN + i) * TM * kWave + j * kWave + lane];
      }
    }
  }
  const bool holder = wk == 0;  // the waves that now hold the tile's sums
  write_tile<BM, BN, TM, TN, SPLIT>(p, acc, smem, holder, wrow_m, wrow_n, m0, n0, rows, shape_n, split, m_tile, n_tile,
                                    OUT);
}

}  // namespace fp8g
