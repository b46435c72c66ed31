// Host helpers shared by the ahead-of-time entry points (fp8gemm.hip) and the
// runtime-specialised ones (jit.cpp): argument checks, the CU budget, the
// dense shape -> tile configuration choice and the split-K workspace layout.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "fp8gemm.h"
#include "gemm_kernel.hpp"  // kMaxSplits, kMaxGroups

namespace fp8g {
namespace host {

inline std::atomic<int> g_cu_limit{0};

inline int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

inline int effective_cus() {
  const int d = device_cus();
  const int lim = g_cu_limit.load();
  return (lim > 0 && lim < d) ? lim : d;
}

// Tag of the split-K arrival counters.  A call that runs to the end leaves
// every counter word it used at (tag, 0), from which the next call with the
// same tag counts with one atomic add per arrival; any other word is
// restarted by its tile's first arrival.  The tag moves on only when a
// launch fails, since a split call whose later launches never ran (a CU
// limit cuts it into several) may leave counts part-way.  As FP32, and as
// either BF16 half, the starting value is a signalling NaN, which no
// partial sum or output of these kernels can hold.
inline std::atomic<unsigned> g_counter_tag{0xFFA5C3E1u};
inline unsigned counter_tag() { return g_counter_tag.load(); }
inline void retire_counter_tag() {
  if (g_counter_tag.fetch_add(1) + 1 == 0) g_counter_tag.fetch_add(1);
}

// Launches a GEMM of `units` work units (one workgroup each): all in one
// launch, or, while a CU limit is in force, in consecutive launches of at
// most that many workgroups, so that at most that many CUs run the GEMM at
// any time (later slices start when earlier ones have drained, in stream
// order).  launch_one(grid) issues one launch of p with p.unit_offset set;
// the first nonzero status it returns stops the sequence.
template <typename Params, typename Launch>
inline int launch_units(Params& p, int64_t units, Launch&& launch_one) {
  p.units = int(units);
  const int lim = g_cu_limit.load();
  const int64_t step = (lim > 0 && lim < device_cus() && units > lim) ? lim : units;
  for (int64_t off = 0; off < units; off += step) {
    p.unit_offset = int(off);
    if (const int st = launch_one(std::min(step, units - off))) {
      if (p.splits > 1) retire_counter_tag();
      return st;
    }
  }
  return 0;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline bool log_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("FP8G_LOG");
    return v && v[0] == '1';
  }();
  return on;
}

inline int launched(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    if (log_enabled()) std::fprintf(stderr, "[fp8gemm] %s launch failed: %s\n", what, hipGetErrorString(e));
    return FP8G_ELAUNCH;
  }
  return FP8G_OK;
}

// Common GEMM shape limits of this version.
inline int check_gemm_shape(int n, int k) {
  if (n < 0 || k < 0) return FP8G_EINVAL;
  if (k == 0 || k % 128 != 0 || k / 128 > fp8g::kMaxGroups) return FP8G_EUNSUPPORTED;
  if (n % 8 != 0) return FP8G_EUNSUPPORTED;
  return FP8G_OK;
}

// (the kernels index a scale row with 32-bit ints)
inline int check_ld(int64_t ld, int64_t rows) {
  if (ld < rows || ld % 4 != 0 || ld < 4 || ld > INT32_MAX) return FP8G_EUNSUPPORTED;
  return FP8G_OK;
}

// ---- dense configuration ---------------------------------------------------
// Kernel shapes: BM tokens x BN outputs per workgroup, wave grid, LDS stages,
// K groups per stage (ku) and waves sharing a sub-tile (wk).  A wave's
// accumulator tile is at most 128 x 64 (128 VGPRs): the promotion FMAs need
// their accumulators in architectural VGPRs.  The large-M shape runs two
// waves per SIMD (eight per workgroup) so that one wave's LDS and barrier
// waits are covered by the other's MFMAs.  m <= 128 is HBM-bound and picks
// among four tile families by the estimate in dense_config.
struct KernelShape {
  int bm, bn, stages, waves, ku;
  int wm, wn, wk;  // wave grid: waves along M and N, and waves sharing a sub-tile
};
enum DenseKind { kBig = 0, kS128N64 = 1, kF64N32 = 2, kF64N64 = 3, kF64N128 = 4, kF128N128 = 5, kKinds = 6 };
constexpr KernelShape kShapes[kKinds] = {
    {256, 256, 2, 8, 1, 4, 2, 1},  // m > 128
    {128, 64, 4, 4, 1, 2, 2, 1},   // m > 128 with few 256 x 256 tiles (split-K)
    {64, 32, 4, 4, 2, 4, 1, 1},    // m <= 128 families
    {64, 64, 4, 8, 2, 2, 2, 2},
    {64, 128, 4, 8, 1, 4, 2, 1},
    {128, 128, 3, 8, 1, 4, 2, 1},
};
constexpr int kSmallFamilies[] = {kF64N32, kF64N64, kF64N128, kF128N128};
// The grouped kernels' shapes: contiguous 256 x 256 tiles (one or two
// 128-row blocks of one group); masked 64-row tiles, so that slots that are
// mostly empty (decode) waste few rows (measured on 16 slots of 256 rows
// holding U{0..256} tokens each: 64 x 128 was 12% faster than 128 x 128,
// and 64 x 256 with 2 x 4 waves and three stages 2-4% faster than 64 x 128,
// alternated four times on one box: the wider tile copies the shared LHS
// rows once per 256 outputs instead of once per 128).
constexpr KernelShape kContiguousShape = {256, 256, 2, 8, 1, 4, 2, 1};
constexpr KernelShape kMaskedShape = {64, 256, 3, 8, 1, 2, 4, 1};

struct DenseConfig {
  int kind, tiles_m, tiles_n, splits, gps;
};

inline int env_int(const char* name, int fallback) {
  const char* v = std::getenv(name);
  return (v && *v) ? std::atoi(v) : fallback;
}

// Split count of a configuration: the K groups are dealt in equal runs, so
// the count is rounded to what those runs give.
inline int whole_splits(int kg, int s) { return int(cdiv(kg, cdiv(kg, std::max(1, std::min(s, kg))))); }

// m <= 128: every workgroup streams its K range of BM LHS rows and BN RHS
// rows through LDS, and the time goes with the busiest CU.  Candidates run
// at most one workgroup per CU (measured: a second round of workgroups
// costs more than any tile choice saves); among them the estimate
//     K groups per workgroup * (BM + BN) * 128 B / 80 GB/s
//     + (when K is split into s) s * 1 us + s * m * n * 8 B / 4 TB/s
// is least: the per-CU copy rate, the fix-up latency and the partial sums'
// round trip through memory, as measured on MI355X.  Over 24 shapes (m in
// 32..128, n 1536..32768, k 512..16384) the pick was within 7% of the best
// of 218 tile configurations x split counts, 1.4% on average.  If no family
// fits in one round, the one with the fewest tiles runs unsplit.
inline void small_m_choice(int m, int n, int kg, int cus, bool allow_split, int* kind, int* splits) {
  double best = 0.0;
  int best_kind = -1, best_splits = 1, fewest_kind = -1;
  int64_t fewest = 0;
  for (int f : kSmallFamilies) {
    const KernelShape& ks = kShapes[f];
    if (m <= 64 && ks.bm > 64) continue;
    const int64_t tiles = cdiv(m, ks.bm) * cdiv(n, ks.bn);
    if (fewest_kind < 0 || tiles < fewest) { fewest = tiles; fewest_kind = f; }
    for (int s0 : {1, 2, 3, 4, 6, 8}) {
      const int s = whole_splits(kg, s0);
      if ((s > 1 && !allow_split) || (s0 > 1 && s == 1) || tiles * s > cus) continue;
      const double t = double(cdiv(kg, s)) * double(ks.bm + ks.bn) * 128.0 / 80e9 +
                       (s > 1 ? 1e-6 * s + double(s) * m * n * 8.0 / 4e12 : 0.0);
      if (best_kind < 0 || t < best) { best = t; best_kind = f; best_splits = s; }
    }
  }
  *kind = best_kind >= 0 ? best_kind : fewest_kind;
  *splits = best_kind >= 0 ? best_splits : 1;
}

inline DenseConfig dense_config(int m, int n, int k, bool allow_split) {
  DenseConfig c{};
  const int cus = effective_cus();
  const int kg = k / 128;
  int splits = 1;
  if (m <= 128) {
    small_m_choice(m, n, kg, cus, allow_split, &c.kind, &splits);
  } else {
    c.kind = kBig;
    // large M but few 256 x 256 tiles: narrower tiles with split-K fill the CUs
    if (cdiv(m, 256) * cdiv(n, 256) < cus / 2) c.kind = kS128N64;
  }
  const int forced = env_int("FP8G_FORCE_CONFIG", -1);  // debugging and tuning only
  if (forced >= 0 && forced < kKinds) c.kind = forced;
  const KernelShape& ks = kShapes[c.kind];
  c.tiles_m = int(cdiv(m, ks.bm));
  c.tiles_n = int(cdiv(n, ks.bn));
  const int64_t tiles = int64_t(c.tiles_m) * c.tiles_n;
  const bool can_split = ks.bm * (ks.bn + 4) * 4 <= ks.stages * ks.ku * (ks.bm + ks.bn) * 128;  // staged tile fits the ring
  if (m > 128 || forced >= 0) {
    // Split only when it at least doubles the workgroup count: each split
    // adds a partial-sum round trip through memory at the end of the kernel.
    splits = 1;
    if (allow_split && can_split && 2 * tiles <= cus + tiles / 2)
      splits = int(std::min<int64_t>(kg, (cus + tiles / 2) / tiles));
  }
  if (allow_split && can_split) {
    // FP8G_SPLITS overrides the split count (tuning only); it never turns
    // split-K on where the workspace or the tile cannot take it
    splits = std::max(1, std::min(std::min(kg, kMaxSplits), env_int("FP8G_SPLITS", splits)));
  } else {
    splits = 1;
  }
  c.gps = int(cdiv(kg, splits));
  c.splits = int(cdiv(kg, c.gps));
  return c;
}

// Workspace of a split configuration: one 8-byte arrival counter per output
// tile (rounded up to 256 bytes), then [splits][m][n] fp32 partial sums.
inline size_t counter_bytes(const DenseConfig& c) {
  return size_t(cdiv(int64_t(c.tiles_m) * c.tiles_n * 8, 256)) * 256;
}

inline size_t dense_workspace(const DenseConfig& c, int m, int n) {
  return c.splits > 1 ? counter_bytes(c) + size_t(c.splits) * size_t(m) * size_t(n) * sizeof(float) : 0;
}

}  // namespace host
}  // namespace fp8g
