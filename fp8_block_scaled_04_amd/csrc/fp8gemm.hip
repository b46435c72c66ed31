// Host side of the C-ABI library libfp8gemm.so (declared in fp8gemm.h):
// argument validation, the shape -> kernel configuration choice, grid sizing
// for the CU budget, and the launches.  Nothing here synchronises or reads
// device memory; every failure the host can detect is returned before any
// launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstdio>
#include <mutex>
#include <vector>

#include "fp8gemm.h"
#include "cast_kernel.hpp"
#include "gemm_kernel.hpp"
#include "host_common.hpp"
#include "dense_launch.hpp"

namespace {

using fp8g::GemmParams;
using fp8g::gemm_kernel;
using fp8g::kContiguous;
using fp8g::kDense;
using fp8g::kMasked;
using namespace fp8g::host;

// Every instantiation below matches its row of kShapes (tile, wave grid,
// ring depth, K groups per stage), kContiguousShape or kMaskedShape.
template <int BM, int BN, int WMW, int WNW, int ST, int MODE, bool SPLIT, int KU = 1, int WK = 1, int FMT = 0>
void launch_gemm(const GemmParams& p, int64_t grid, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WMW, WNW, ST, MODE, SPLIT, KU, WK, FMT>), dim3(unsigned(grid)),
                     dim3(64 * WMW * WNW * WK), 0, s, p);
}

// The dense GEMM kernels are instantiated in dense_launch.hip, one object per
// operand-format pair (FMT: bit 0 = LHS in E5M2, bit 1 = RHS in E5M2).
int launch_dense_fmt(bool split, int fmt, int kind, const GemmParams& p, int64_t grid, hipStream_t s) {
  switch (fmt) {
    case 1: return fp8g::host::launch_dense_kind<1>(split, kind, p, grid, s);
    case 2: return fp8g::host::launch_dense_kind<2>(split, kind, p, grid, s);
    case 3: return fp8g::host::launch_dense_kind<3>(split, kind, p, grid, s);
    default: return fp8g::host::launch_dense_kind<0>(split, kind, p, grid, s);
  }
}

template <int FMT>
void launch_cast_1x128(const void* x, int x_dtype, bool pair, dim3 grid, hipStream_t s, int m, int k, uint8_t* q,
                       float* scales, int64_t scales_ld) {
  if (x_dtype == FP8G_F32) {
    if (pair)
      hipLaunchKernelGGL((fp8g::cast_1x128_kernel<float, 2, FMT>), grid, dim3(256), 0, s,
                         static_cast<const float*>(x), m, k, q, scales, scales_ld);
    else
      hipLaunchKernelGGL((fp8g::cast_1x128_kernel<float, 1, FMT>), grid, dim3(256), 0, s,
                         static_cast<const float*>(x), m, k, q, scales, scales_ld);
  } else {
    if (pair)
      hipLaunchKernelGGL((fp8g::cast_1x128_kernel<uint16_t, 2, FMT>), grid, dim3(256), 0, s,
                         static_cast<const uint16_t*>(x), m, k, q, scales, scales_ld);
    else
      hipLaunchKernelGGL((fp8g::cast_1x128_kernel<uint16_t, 1, FMT>), grid, dim3(256), 0, s,
                         static_cast<const uint16_t*>(x), m, k, q, scales, scales_ld);
  }
}

// Host checks shared by the dense entry points (everything the host can
// check, before any launch); fmt receives the operand-format code.
int check_dense_args(const uint8_t* lhs, int lhs_format, const float* lhs_scales, int64_t lhs_scales_ld,
                     const uint8_t* rhs, int rhs_format, const float* rhs_scales, const uint16_t* out, int m, int n,
                     int k, const void* workspace, int* fmt) {
  if (m < 0) return FP8G_EINVAL;
  if ((lhs_format != FP8G_E4M3 && lhs_format != FP8G_E5M2) || (rhs_format != FP8G_E4M3 && rhs_format != FP8G_E5M2))
    return FP8G_EINVAL;
  *fmt = (lhs_format == FP8G_E5M2 ? 1 : 0) | (rhs_format == FP8G_E5M2 ? 2 : 0);
  if (int st = check_gemm_shape(n, k)) return st;
  if (m == 0 || n == 0) return FP8G_OK;
  if (!lhs || !lhs_scales || !rhs || !rhs_scales || !out) return FP8G_EINVAL;
  if (!aligned16(lhs) || !aligned16(lhs_scales) || !aligned16(rhs) || !aligned16(rhs_scales) ||
      !aligned16(out) || (workspace && !aligned16(workspace)))
    return FP8G_EINVAL;
  return check_ld(lhs_scales_ld, m);
}

// The dense GEMM of checked arguments (m, n > 0): configuration, split-K
// workspace layout, launches.
int run_dense_gemm(const uint8_t* lhs, int fmt, const float* lhs_scales, int64_t lhs_scales_ld, const uint8_t* rhs,
                   const float* rhs_scales, uint16_t* out, int m, int n, int k, void* workspace,
                   size_t workspace_bytes, void* stream) {
  DenseConfig c = dense_config(m, n, k, true);
  if (c.splits > 1 && (!workspace || workspace_bytes < dense_workspace(c, m, n)))
    c = dense_config(m, n, k, false);

  GemmParams p{};
  p.a = lhs; p.sa = lhs_scales; p.b = rhs; p.sb = rhs_scales; p.out = out;
  if (c.splits > 1) {
    p.tile_counters = static_cast<unsigned long long*>(workspace);
    p.partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + counter_bytes(c));
    p.tag = counter_tag();
  }
  p.sa_ld = lhs_scales_ld;
  p.m = m; p.n = n; p.k = k; p.kg = k / 128; p.nb = int(cdiv(n, 128));
  p.tiles_m = c.tiles_m; p.tiles_n = c.tiles_n; p.splits = c.splits; p.groups_per_split = c.gps;
  const int64_t grid = int64_t(c.tiles_m) * c.tiles_n * c.splits;
  if (grid > 0x7fffffff) return FP8G_EUNSUPPORTED;
  auto s = static_cast<hipStream_t>(stream);
  if (log_enabled())
    std::fprintf(stderr, "[fp8gemm] dense m=%d n=%d k=%d kind=%d tiles=%dx%d splits=%d grid=%lld\n", m, n, k,
                 c.kind, c.tiles_m, c.tiles_n, c.splits, (long long)grid);
  return launch_units(p, grid, [&](int64_t g) {
    if (const int st = launch_dense_fmt(c.splits > 1, fmt, c.kind, p, g, s)) return st;  // before any launch
    return launched("gemm");
  });
}

// ---- scratch of the no-allocation entry point --------------------------------
// Split-K arrival counters and partial sums of fp8_gemm_nt_noalloc live in
// this file-scope device array: one copy per device, allocated when the
// library's code is loaded on that device and held until the process ends.
// In host code `scratch` only names the symbol; its device address on each
// device comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is handed to kernels.  The
// counters carry a tag, so nothing in it needs clearing.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int noalloc_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return FP8G_ELAUNCH;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      if (log_enabled()) std::fprintf(stderr, "[fp8gemm] device %d: no address for the scratch array\n", dev);
      return FP8G_ELAUNCH;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return FP8G_OK;
}

}  // namespace

extern "C" {

const char* fp8_status_string(int status) {
  switch (status) {
    case FP8G_OK: return "ok";
    case FP8G_EINVAL: return "invalid argument";
    case FP8G_EUNSUPPORTED: return "unsupported shape or layout";
    case FP8G_ELAUNCH: return "kernel launch failed";
    case FP8G_ESCRATCH: return "problem needs more scratch than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

int fp8_set_num_cus(int num_cus) {
  const int prev = g_cu_limit.load();
  g_cu_limit.store(num_cus < 0 ? 0 : num_cus);
  return prev;
}

int fp8_get_num_cus(void) { return effective_cus(); }

size_t fp8_gemm_workspace_bytes(int m, int n, int k, int num_groups) {
  (void)num_groups;
  if (m <= 0 || n <= 0 || k <= 0 || k % 128 != 0) return 0;
  const DenseConfig c = dense_config(m, n, k, true);
  return dense_workspace(c, m, n);
}

int fp8_gemm_describe(int m, int n, int k, char* buf, size_t len) {
  if (!buf || len == 0 || m < 0) return FP8G_EINVAL;
  if (const int st = check_gemm_shape(n, k)) return st;
  if (m == 0 || n == 0) {
    std::snprintf(buf, len, "empty");
    return FP8G_OK;
  }
  const DenseConfig c = dense_config(m, n, k, true);
  const KernelShape& ks = kShapes[c.kind];
  std::snprintf(buf, len, "tile=%dx%d waves=%d stages=%d ku=%d splits=%d grid=%lld", ks.bm, ks.bn, ks.waves,
                ks.stages, ks.ku, c.splits, (long long)(int64_t(c.tiles_m) * c.tiles_n * c.splits));
  return FP8G_OK;
}

int fp8_gemm_schedule(int mode, int m, int n, int k, int num_groups, const int32_t* group_data, int32_t* units,
                      int capacity) {
  using namespace fp8g;
  if (m < 0 || num_groups < 0 || capacity < 0 || (capacity > 0 && !units)) return FP8G_EINVAL;
  if (mode != FP8G_JIT_DENSE && mode != FP8G_JIT_CONTIGUOUS && mode != FP8G_JIT_MASKED) return FP8G_EINVAL;
  if (const int st = check_gemm_shape(n, k)) return st;
  if (mode == FP8G_JIT_CONTIGUOUS && m % 128 != 0) return FP8G_EUNSUPPORTED;
  if (m == 0 || n == 0 || (mode != FP8G_JIT_DENSE && num_groups == 0)) return 0;
  if (mode != FP8G_JIT_DENSE && !group_data) return FP8G_EINVAL;

  // The launch parameters the entry point would use (the dense one with a
  // large enough workspace), then every workgroup of every launch that
  // launch_units makes, decoded as the kernel decodes it.
  GemmParams p{};
  int bm = 0;
  int64_t grid = 0;
  if (mode == FP8G_JIT_DENSE) {
    const DenseConfig c = dense_config(m, n, k, true);
    bm = kShapes[c.kind].bm;
    p.tiles_m = c.tiles_m; p.tiles_n = c.tiles_n; p.splits = c.splits;
    grid = int64_t(c.tiles_m) * c.tiles_n * c.splits;
  } else if (mode == FP8G_JIT_CONTIGUOUS) {
    bm = kContiguousShape.bm;
    p.tiles_m = m / 128; p.tiles_n = int(cdiv(n, kContiguousShape.bn)); p.splits = 1;
    grid = int64_t(p.tiles_m) * p.tiles_n;
  } else {
    bm = kMaskedShape.bm;
    p.tiles_m = int(cdiv(m, bm)); p.tiles_n = int(cdiv(n, kMaskedShape.bn)); p.splits = 1;
    grid = int64_t(p.tiles_m) * p.tiles_n * num_groups;
  }
  if (grid > 0x7fffffff) return FP8G_EUNSUPPORTED;

  // contiguous: the wave-wide scan, lane by lane (the kernel's steps, the
  // shuffles replaced by loops over the 64 lanes)
  const int nblk = m / 128;
  ContigScan cs[kWave] = {};
  int contig_tiles = 0;
  if (mode == FP8G_JIT_CONTIGUOUS) {
    int run_max = -1;
    for (int lane = 0; lane < kWave; ++lane) {
      contig_chunk(lane, nblk, cs[lane].lo, cs[lane].hi);
      cs[lane].in_rs = lane == 0 ? -1 : run_max;  // max over lanes < this one
      run_max = std::max(run_max, contig_last_run_start(group_data, cs[lane].lo, cs[lane].hi));
    }
    for (int lane = 0; lane < kWave; ++lane) {
      cs[lane].count = contig_count(group_data, cs[lane].lo, cs[lane].hi, cs[lane].in_rs);
      cs[lane].base = contig_tiles;
      contig_tiles += cs[lane].count;
    }
  }
  // masked: the live units of every group, numbered group by group
  std::vector<int> first_unit;
  int masked_total = 0;
  if (mode == FP8G_JIT_MASKED) {
    for (int g = 0; g < num_groups; ++g) {
      first_unit.push_back(masked_total);
      masked_total += masked_live_tiles(group_data[g], m, bm) * p.tiles_n;
    }
  }

  int64_t written = 0;
  auto record = [&](int taken, int group, int row0, int rows, int n_tile, int split) {
    if (written < capacity) {
      int32_t* r = units + 6 * written;
      r[0] = taken; r[1] = group; r[2] = row0; r[3] = rows; r[4] = n_tile; r[5] = split;
    }
    ++written;
  };
  launch_units(p, grid, [&](int64_t g) {
    for (int64_t b = 0; b < g; ++b) {
      const int bid = int(b) + p.unit_offset;
      if (mode == FP8G_JIT_DENSE) {
        int mt, nt, sp;
        dense_tile(p.unit_offset + xcd_logical(int(b), int(g)), p.tiles_m, p.tiles_n, p.splits, mt, nt, sp);
        record(1, 0, mt * bm, std::min(bm, m - mt * bm), nt, sp);
      } else if (mode == FP8G_JIT_CONTIGUOUS) {
        if (bid >= contig_tiles * p.tiles_n) { record(0, -1, 0, 0, 0, 0); continue; }
        int t, nt, sp;
        dense_tile(xcd_logical(bid, contig_tiles * p.tiles_n), contig_tiles, p.tiles_n, 1, t, nt, sp);
        int block = -1;
        for (int lane = 0; lane < kWave && block < 0; ++lane)
          block = contig_find(group_data, cs[lane].lo, cs[lane].hi, cs[lane].in_rs, cs[lane].base, cs[lane].count, t);
        if (block < 0) { record(0, -2, 0, 0, 0, 0); continue; }  // no lane holds the tile: a scheduler bug
        record(1, block_group(group_data, block), 128 * block, 128 * contig_tile_blocks(group_data, nblk, block), nt,
               0);
      } else {
        const int L = xcd_logical(bid, masked_total);
        if (L < 0) { record(0, -1, 0, 0, 0, 0); continue; }
        const int g = int(std::upper_bound(first_unit.begin(), first_unit.end(), L) - first_unit.begin()) - 1;
        const int mt = masked_live_tiles(group_data[g], m, bm);
        const int r = L - first_unit[g];
        const int rows = std::min(std::max(group_data[g], 0), m);
        const int row0 = (r % mt) * bm;
        record(1, g, row0, std::min(bm, rows - row0), r / mt, 0);
      }
    }
    return 0;
  });
  return int(written);
}

int fp8_gemm_nt(const uint8_t* lhs, const float* lhs_scales, int64_t lhs_scales_ld,
                const uint8_t* rhs, const float* rhs_scales, uint16_t* out, int m, int n, int k,
                void* workspace, size_t workspace_bytes, void* stream) {
  return fp8_gemm_nt_fmt(lhs, FP8G_E4M3, lhs_scales, lhs_scales_ld, rhs, FP8G_E4M3, rhs_scales, out, m, n, k,
                         workspace, workspace_bytes, stream);
}

int fp8_gemm_nt_fmt(const uint8_t* lhs, int lhs_format, const float* lhs_scales, int64_t lhs_scales_ld,
                    const uint8_t* rhs, int rhs_format, const float* rhs_scales, uint16_t* out, int m, int n,
                    int k, void* workspace, size_t workspace_bytes, void* stream) {
  int fmt = 0;
  if (const int st = check_dense_args(lhs, lhs_format, lhs_scales, lhs_scales_ld, rhs, rhs_format, rhs_scales, out,
                                      m, n, k, workspace, &fmt))
    return st;
  if (m == 0 || n == 0) return FP8G_OK;
  return run_dense_gemm(lhs, fmt, lhs_scales, lhs_scales_ld, rhs, rhs_scales, out, m, n, k, workspace,
                        workspace_bytes, stream);
}

int fp8_gemm_nt_noalloc(const uint8_t* lhs, const float* lhs_scales, int64_t lhs_scales_ld, const uint8_t* rhs,
                        const float* rhs_scales, uint16_t* out, int m, int n, int k, void* stream) {
  int fmt = 0;
  if (const int st = check_dense_args(lhs, FP8G_E4M3, lhs_scales, lhs_scales_ld, rhs, FP8G_E4M3, rhs_scales, out, m,
                                      n, k, nullptr, &fmt))
    return st;
  if (m == 0 || n == 0) return FP8G_OK;
  // the configuration fp8_gemm_nt picks with a large enough workspace
  const DenseConfig c = dense_config(m, n, k, true);
  if (dense_workspace(c, m, n) > kNoAllocScratchBytes) {
    if (log_enabled())
      std::fprintf(stderr, "[fp8gemm] no-allocation GEMM m=%d n=%d k=%d needs %zu scratch bytes, above %zu\n", m, n,
                   k, dense_workspace(c, m, n), kNoAllocScratchBytes);
    return FP8G_ESCRATCH;
  }
  void* ws = nullptr;
  if (const int st = noalloc_scratch(&ws)) return st;
  return run_dense_gemm(lhs, fmt, lhs_scales, lhs_scales_ld, rhs, rhs_scales, out, m, n, k, ws,
                        kNoAllocScratchBytes, stream);
}

int fp8_grouped_gemm_contiguous(const uint8_t* lhs, const float* lhs_scales, int64_t lhs_scales_ld,
                                const uint8_t* rhs, const float* rhs_scales, uint16_t* out,
                                const int32_t* m_indices, int m_total, int n, int k, int num_groups,
                                void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace; (void)workspace_bytes;
  if (m_total < 0 || num_groups < 0) return FP8G_EINVAL;
  if (int st = check_gemm_shape(n, k)) return st;
  if (m_total % 128 != 0) return FP8G_EUNSUPPORTED;
  if (m_total == 0 || n == 0 || num_groups == 0) return FP8G_OK;
  if (!lhs || !lhs_scales || !rhs || !rhs_scales || !out || !m_indices) return FP8G_EINVAL;
  if (!aligned16(lhs) || !aligned16(lhs_scales) || !aligned16(rhs) || !aligned16(rhs_scales) ||
      !aligned16(out) || !aligned16(m_indices))
    return FP8G_EINVAL;
  if (int st = check_ld(lhs_scales_ld, m_total)) return st;

  GemmParams p{};
  p.a = lhs; p.sa = lhs_scales; p.b = rhs; p.sb = rhs_scales; p.out = out;
  p.m_indices = m_indices;
  p.sa_ld = lhs_scales_ld;
  p.m = m_total; p.n = n; p.k = k; p.kg = k / 128; p.nb = int(cdiv(n, 128));
  // Tiles are one or two 128-row blocks of one group (the kernel finds them
  // from m_indices); there are at most as many tiles as blocks.
  p.tiles_m = m_total / 128; p.tiles_n = int(cdiv(n, 256)); p.splits = 1; p.groups_per_split = p.kg;
  const int64_t grid = int64_t(p.tiles_m) * p.tiles_n;
  if (grid > 0x7fffffff) return FP8G_EUNSUPPORTED;
  if (log_enabled())
    std::fprintf(stderr, "[fp8gemm] contiguous M=%d n=%d k=%d G=%d grid<=%lld\n", m_total, n, k, num_groups,
                 (long long)grid);
  return launch_units(p, grid, [&](int64_t g) {
    launch_gemm<256, 256, 4, 2, 2, kContiguous, false>(p, g, static_cast<hipStream_t>(stream));
    return launched("contiguous gemm");
  });
}

int fp8_grouped_gemm_masked(const uint8_t* lhs, const float* lhs_scales, int64_t lhs_scales_ld,
                            const uint8_t* rhs, const float* rhs_scales, uint16_t* out,
                            const int32_t* masked_m, int num_groups, int max_m, int n, int k,
                            void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace; (void)workspace_bytes;
  if (num_groups < 0 || max_m < 0) return FP8G_EINVAL;
  if (int st = check_gemm_shape(n, k)) return st;
  if (num_groups == 0 || max_m == 0 || n == 0) return FP8G_OK;
  if (!lhs || !lhs_scales || !rhs || !rhs_scales || !out || !masked_m) return FP8G_EINVAL;
  if (!aligned16(lhs) || !aligned16(lhs_scales) || !aligned16(rhs) || !aligned16(rhs_scales) ||
      !aligned16(out) || !aligned16(masked_m))
    return FP8G_EINVAL;
  if (int st = check_ld(lhs_scales_ld, max_m)) return st;

  GemmParams p{};
  p.a = lhs; p.sa = lhs_scales; p.b = rhs; p.sb = rhs_scales; p.out = out;
  p.masked_m = masked_m;
  p.sa_ld = lhs_scales_ld;
  p.m = max_m; p.n = n; p.k = k; p.kg = k / 128; p.nb = int(cdiv(n, 128));
  // The grid covers every possible unit; the kernel hands the live ones
  // (row tiles below each group's count) to the first workgroups of each
  // XCD and the rest exit at once.  The row tiles that share an RHS tile run
  // together on one XCD, so after the first they read it from L2.
  p.tiles_m = int(cdiv(max_m, kMaskedShape.bm)); p.tiles_n = int(cdiv(n, kMaskedShape.bn)); p.splits = 1;
  p.groups_per_split = p.kg;
  const int64_t grid = int64_t(p.tiles_m) * p.tiles_n * num_groups;
  if (grid > 0x7fffffff) return FP8G_EUNSUPPORTED;
  if (log_enabled())
    std::fprintf(stderr, "[fp8gemm] masked G=%d max_m=%d n=%d k=%d grid=%lld\n", num_groups, max_m, n, k,
                 (long long)grid);
  return launch_units(p, grid, [&](int64_t g) {
    launch_gemm<kMaskedShape.bm, kMaskedShape.bn, kMaskedShape.wm, kMaskedShape.wn, kMaskedShape.stages, kMasked,
                false>(p, g, static_cast<hipStream_t>(stream));
    return launched("masked gemm");
  });
}

int fp8_cast_per_token_group(const void* x, int x_dtype, int m, int k, uint8_t* q, float* scales,
                             int64_t scales_ld, void* stream) {
  return fp8_cast_per_token_group_fmt(x, x_dtype, FP8G_E4M3, m, k, q, scales, scales_ld, stream);
}

int fp8_cast_per_token_group_fmt(const void* x, int x_dtype, int q_format, int m, int k, uint8_t* q,
                                 float* scales, int64_t scales_ld, void* stream) {
  if (q_format != FP8G_E4M3 && q_format != FP8G_E5M2) return FP8G_EINVAL;
  if (m < 0 || k < 0) return FP8G_EINVAL;
  if (x_dtype != FP8G_F32 && x_dtype != FP8G_BF16) return FP8G_EINVAL;
  if (k % 8 != 0) return FP8G_EUNSUPPORTED;
  if (m == 0 || k == 0) return FP8G_OK;
  if (!x || !q || !scales) return FP8G_EINVAL;
  if (!aligned16(x) || !aligned16(q) || !aligned16(scales)) return FP8G_EINVAL;
  if (scales_ld < m) return FP8G_EUNSUPPORTED;
  const int64_t kg = cdiv(k, 128);
  if (kg > 65535) return FP8G_EUNSUPPORTED;  // keeps the kernel's 32-bit column arithmetic in range
  // two K groups per workgroup once there are many (long rows of a large
  // activation): fewer, longer workgroups keep more loads in flight
  const bool pair = kg >= 64;
  const int64_t blocks = cdiv(m, 16) * (pair ? cdiv(kg, 2) : kg);
  if (blocks > 0x7fffffff) return FP8G_EUNSUPPORTED;
  const dim3 grid{unsigned(blocks)};
  auto s = static_cast<hipStream_t>(stream);
  if (q_format == FP8G_E5M2)
    launch_cast_1x128<fp8g::kFmtE5M2>(x, x_dtype, pair, grid, s, m, k, q, scales, scales_ld);
  else
    launch_cast_1x128<fp8g::kFmtE4M3>(x, x_dtype, pair, grid, s, m, k, q, scales, scales_ld);
  return launched("per-token-group cast");
}

int fp8_cast_per_block(const float* w, int n, int k, uint8_t* q, float* scales, void* stream) {
  return fp8_cast_per_block_fmt(w, FP8G_E4M3, n, k, q, scales, stream);
}

int fp8_cast_per_block_fmt(const float* w, int q_format, int n, int k, uint8_t* q, float* scales, void* stream) {
  if (q_format != FP8G_E4M3 && q_format != FP8G_E5M2) return FP8G_EINVAL;
  if (n < 0 || k < 0) return FP8G_EINVAL;
  if (k % 4 != 0) return FP8G_EUNSUPPORTED;
  if (n == 0 || k == 0) return FP8G_OK;
  if (!w || !q || !scales) return FP8G_EINVAL;
  if (!aligned16(w) || !aligned16(q) || !aligned16(scales)) return FP8G_EINVAL;
  const int64_t kg = cdiv(k, 128), nb = cdiv(n, 128);
  if (kg > 65535 || nb * kg > 0x7fffffff) return FP8G_EUNSUPPORTED;
  const dim3 grid{unsigned(nb * kg)};
  if (q_format == FP8G_E5M2)
    hipLaunchKernelGGL(fp8g::cast_128x128_kernel<fp8g::kFmtE5M2>, grid, dim3(256), 0,
                       static_cast<hipStream_t>(stream), w, n, k, q, scales, int(kg));
  else
    hipLaunchKernelGGL(fp8g::cast_128x128_kernel<fp8g::kFmtE4M3>, grid, dim3(256), 0,
                       static_cast<hipStream_t>(stream), w, n, k, q, scales, int(kg));
  return launched("block cast");
}

}  // extern "C"
