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

inline int check_ld(int64_t ld, int64_t rows) {
  if (ld < rows || ld % 4 != 0 || ld < 4) return FP8G_EUNSUPPORTED;
  return FP8G_OK;
}

// ---- dense configuration ---------------------------------------------------
// Kernel shapes: BM tokens x BN outputs per workgroup, wave grid, LDS stages,
// K groups per stage (ku) and waves sharing a sub-tile (wk).  A wave's
// accumulator tile is at most 128 x 64 (128 VGPRs): the promotion FMAs need
// their accumulators in architectural VGPRs.  The large-M shape runs two
// waves per SIMD (eight per workgroup) so that one wave's LDS and barrier
// waits are covered by the other's MFMAs.  Small-M shapes are HBM-bound:
// narrow N tiles give enough workgroups; with few tiles per CU each wave
// multiplies whole 64 x 32 tiles of its own K groups (ku = wk = 4), which
// keeps more independent MFMAs in flight per stage; with many tiles per CU,
// several small workgroups share a CU instead.  When the tile count would
// leave CUs idle, K is split across workgroups; the last workgroup to finish
// a tile adds the partial sums in split order.
struct KernelShape {
  int bm, bn, stages, waves, ku;
  int wm, wn, wk;  // wave grid: waves along M and N, and waves sharing a sub-tile
};
enum DenseKind { kS64N64 = 0, kS64N128 = 1, kS128N64 = 2, kS128N128 = 3, kBig = 4, kMid = 5, kS64N32 = 6,
                 kS128N32 = 7, kS64N32K4 = 8, kS128N32K2 = 9, kKinds = 10 };
constexpr KernelShape kShapes[kKinds] = {
    {64, 64, 4, 4, 1, 1, 4, 1},    // m <= 64
    {64, 128, 4, 4, 1, 1, 4, 1},
    {128, 64, 4, 4, 1, 2, 2, 1},   // 64 < m <= 128
    {128, 128, 3, 4, 1, 2, 2, 1},
    {256, 256, 2, 8, 1, 4, 2, 1},  // m > 128
    {256, 128, 3, 4, 1, 2, 2, 1},
    {64, 32, 4, 4, 1, 2, 2, 1},
    {128, 32, 4, 4, 1, 4, 1, 1},
    {64, 32, 3, 4, 4, 1, 1, 4},    // m <= 64, few tiles per CU: four waves, four K groups per stage
    {128, 32, 3, 4, 2, 2, 1, 2},   // 64 < m <= 128, few tiles per CU
};
// The grouped kernels' shapes: contiguous 256 x 256 tiles (one or two
// 128-row blocks of one group), masked 128 x 128 tiles.
constexpr KernelShape kContiguousShape = {256, 256, 2, 8, 1, 4, 2, 1};
constexpr KernelShape kMaskedShape = {128, 128, 4, 4, 1, 2, 2, 1};
constexpr int kMaxSplits = 8;  // the split-K fix-up adds at most this many partials

struct DenseConfig {
  int kind, tiles_m, tiles_n, splits, gps;
};

inline int env_int(const char* name, int fallback) {
  const char* v = std::getenv(name);
  return (v && *v) ? std::atoi(v) : fallback;
}

inline DenseConfig dense_config(int m, int n, int k, bool allow_split, bool all_kinds = true) {
  DenseConfig c{};
  const int cus0 = effective_cus();
  // few 32-column tiles per CU: the K-group-sharing shapes; many: the plain ones
  const bool few = cdiv(n, 32) < 2 * int64_t(cus0);
  c.kind = m <= 64 ? (few ? kS64N32K4 : kS64N32) : (m <= 128 ? (few ? kS128N32K2 : kS128N32) : kBig);
  // large M but few 256 x 256 tiles: narrower tiles with split-K fill the CUs
  if (c.kind == kBig && cdiv(m, 256) * cdiv(n, 256) < cus0 / 2) c.kind = kS128N64;
  const int forced = env_int("FP8G_FORCE_CONFIG", -1);  // debugging and tuning only
  if (forced >= 0 && forced < kKinds && all_kinds) c.kind = forced;
  const KernelShape& ks = kShapes[c.kind];
  c.tiles_m = int(cdiv(m, ks.bm));
  c.tiles_n = int(cdiv(n, ks.bn));
  const int kg = k / 128;
  c.splits = 1;
  c.gps = kg;
  const int64_t tiles = int64_t(c.tiles_m) * c.tiles_n;
  const int cus = effective_cus();
  const bool can_split = ks.bm * (ks.bn + 4) * 4 <= ks.stages * ks.ku * (ks.bm + ks.bn) * 128;  // staged tile fits the ring
  // Split only when it at least doubles the workgroup count: each split
  // adds a partial-sum round trip through memory at the end of the kernel.
  if (allow_split && can_split && 2 * tiles <= cus + tiles / 2) {
    int s = int(std::min<int64_t>(kg, (cus + tiles / 2) / tiles));
    s = std::max(1, std::min(std::min(kg, kMaxSplits), env_int("FP8G_SPLITS", s)));
    c.gps = int(cdiv(kg, s));
    c.splits = int(cdiv(kg, c.gps));
  }
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

// Per-call tag of the split-K arrival counters (never 0).
inline std::atomic<unsigned> g_epoch{0};
inline unsigned next_epoch() {
  unsigned e = g_epoch.fetch_add(1) + 1;
  if (e == 0) e = g_epoch.fetch_add(1) + 1;
  return e;
}

}  // namespace host
}  // namespace fp8g
