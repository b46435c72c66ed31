// Host side of the MoE layout entry points of libfp8gemm.so (declared in
// fp8gemm.h): validation, workspace accounting and launches.  Nothing here
// synchronises or reads device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "fp8gemm.h"
#include "moe_kernel.hpp"

namespace {

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }
bool aligned(const void* p, unsigned a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int launched() { return hipGetLastError() == hipSuccess ? FP8G_OK : FP8G_ELAUNCH; }

int64_t chunks(int num_tokens) { return cdiv64(num_tokens, fp8g::kMoeChunk); }

int check_routing(const int32_t* expert_idx, int num_tokens, int num_groups) {
  if (num_tokens < 0 || num_groups < 1) return FP8G_EINVAL;
  if (num_groups > fp8g::kMoeMaxGroups) return FP8G_EUNSUPPORTED;
  if (num_tokens > 0 && !expert_idx) return FP8G_EINVAL;
  if (expert_idx && !aligned(expert_idx, 4)) return FP8G_EINVAL;
  return FP8G_OK;
}

// Counting passes shared by both layouts: per-chunk histograms, then the
// scan (which also writes counts and, per layout, offsets or masked counts).
void count_and_scan(const int32_t* expert_idx, int T, int G, int32_t* hist, int32_t* counts, int32_t* offsets,
                    int32_t* masked_m, int max_m, hipStream_t s) {
  const int64_t B = chunks(T);
  if (B > 0) hipLaunchKernelGGL(fp8g::moe_hist_kernel, dim3(unsigned(B)), dim3(256), 0, s, expert_idx, T, G, hist);
  hipLaunchKernelGGL(fp8g::moe_scan_kernel, dim3(1), dim3(1024), 0, s, hist, int(B), G, counts, offsets, masked_m,
                     max_m);
}

}  // namespace

extern "C" {

int fp8_moe_contiguous_rows(int num_tokens, int num_groups) {
  if (num_tokens < 0 || num_groups < 1) return -1;
  const int64_t rows = cdiv64(int64_t(num_tokens) + int64_t(num_groups) * (fp8g::kMoeAlign - 1), fp8g::kMoeAlign) *
                       fp8g::kMoeAlign;
  return rows > 0x7fffffff ? -1 : int(rows);
}

size_t fp8_moe_layout_workspace_bytes(int num_tokens, int num_groups) {
  if (num_tokens < 0 || num_groups < 1) return 0;
  const size_t bytes = size_t(chunks(num_tokens)) * size_t(num_groups) * sizeof(int32_t);
  return bytes > 0 ? bytes : 4;
}

int fp8_moe_layout_contiguous(const int32_t* expert_idx, int num_tokens, int num_groups, int32_t* counts,
                              int32_t* offsets, int32_t* dst_row, int32_t* m_indices, int m_rows, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (int st = check_routing(expert_idx, num_tokens, num_groups)) return st;
  if (!counts || !offsets || !m_indices || (num_tokens > 0 && !dst_row) || !workspace) return FP8G_EINVAL;
  if (!aligned(counts, 4) || !aligned(offsets, 4) || !aligned(m_indices, 4) || (dst_row && !aligned(dst_row, 4)) ||
      !aligned(workspace, 4))
    return FP8G_EINVAL;
  const int need_rows = fp8_moe_contiguous_rows(num_tokens, num_groups);
  if (need_rows < 0) return FP8G_EUNSUPPORTED;
  if (m_rows < need_rows) return FP8G_EINVAL;
  if (workspace_bytes < fp8_moe_layout_workspace_bytes(num_tokens, num_groups)) return FP8G_EINVAL;
  auto s = static_cast<hipStream_t>(stream);
  if (num_tokens <= fp8g::kMoeSmallRounds * 1024) {  // one workgroup does it all
    hipLaunchKernelGGL(fp8g::moe_layout_small_kernel<true>, dim3(1), dim3(1024), 0, s, expert_idx, num_tokens,
                       num_groups, 0, counts, offsets, dst_row, m_indices, m_rows, nullptr);
    return launched();
  }
  auto* hist = static_cast<int32_t*>(workspace);
  count_and_scan(expert_idx, num_tokens, num_groups, hist, counts, offsets, nullptr, 0, s);
  // destinations and m_indices in one launch (num_tokens > 4096 here, so B > 0)
  const int64_t B = chunks(num_tokens);
  hipLaunchKernelGGL(fp8g::moe_dest_kernel<true>, dim3(unsigned(B)), dim3(1024), 0, s, expert_idx, num_tokens,
                     num_groups, hist, offsets, 0, dst_row, m_indices, m_rows);
  return launched();
}

int fp8_moe_layout_masked(const int32_t* expert_idx, int num_tokens, int num_groups, int max_m, int32_t* counts,
                          int32_t* dst_row, int32_t* masked_m, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (int st = check_routing(expert_idx, num_tokens, num_groups)) return st;
  if (max_m < 0) return FP8G_EINVAL;
  if (!counts || !masked_m || (num_tokens > 0 && !dst_row) || !workspace) return FP8G_EINVAL;
  if (!aligned(counts, 4) || !aligned(masked_m, 4) || (dst_row && !aligned(dst_row, 4)) || !aligned(workspace, 4))
    return FP8G_EINVAL;
  if (int64_t(num_groups) * max_m > 0x7fffffff) return FP8G_EUNSUPPORTED;
  if (workspace_bytes < fp8_moe_layout_workspace_bytes(num_tokens, num_groups)) return FP8G_EINVAL;
  auto s = static_cast<hipStream_t>(stream);
  if (num_tokens <= fp8g::kMoeSmallRounds * 1024) {  // one workgroup does it all
    hipLaunchKernelGGL(fp8g::moe_layout_small_kernel<false>, dim3(1), dim3(1024), 0, s, expert_idx, num_tokens,
                       num_groups, max_m, counts, nullptr, dst_row, nullptr, 0, masked_m);
    return launched();
  }
  auto* hist = static_cast<int32_t*>(workspace);
  count_and_scan(expert_idx, num_tokens, num_groups, hist, counts, nullptr, masked_m, max_m, s);
  const int64_t B = chunks(num_tokens);
  if (B > 0)
    hipLaunchKernelGGL(fp8g::moe_dest_kernel<false>, dim3(unsigned(B)), dim3(1024), 0, s, expert_idx, num_tokens,
                       num_groups, hist, nullptr, max_m, dst_row, nullptr, 0);
  return launched();
}

int fp8_moe_scatter_rows(const uint8_t* q, const float* scales, int64_t scales_ld, int num_tokens, int k,
                         const int32_t* dst_row, int rows_per_group, int out_rows, uint8_t* q_out,
                         float* scales_out, int64_t scales_out_ld, void* stream) {
  if (num_tokens < 0 || k < 0 || out_rows < 0 || rows_per_group < 1) return FP8G_EINVAL;
  if (k % 16 != 0) return FP8G_EUNSUPPORTED;
  if (num_tokens == 0 || k == 0 || out_rows == 0) return FP8G_OK;
  if (!q || !scales || !dst_row || !q_out || !scales_out) return FP8G_EINVAL;
  if (!aligned(q, 16) || !aligned(q_out, 16) || !aligned(scales, 4) || !aligned(scales_out, 4) ||
      !aligned(dst_row, 4))
    return FP8G_EINVAL;
  if (scales_ld < num_tokens || scales_out_ld < rows_per_group || out_rows % rows_per_group != 0)
    return FP8G_EINVAL;
  // rows: four tokens per workgroup; scales: 256 tokens x kMoeScaleGroups K groups per workgroup
  const int64_t row_blocks = cdiv64(num_tokens, 4);
  const int64_t grid = row_blocks + cdiv64(num_tokens, 256) * cdiv64(cdiv64(k, 128), fp8g::kMoeScaleGroups);
  if (grid > 0x7fffffff) return FP8G_EUNSUPPORTED;
  hipLaunchKernelGGL(fp8g::moe_scatter_kernel, dim3(unsigned(grid)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     q, scales, scales_ld, num_tokens, k, dst_row, rows_per_group, out_rows, q_out, scales_out,
                     scales_out_ld, int(row_blocks));
  return launched();
}

int fp8_moe_gather_rows(const uint16_t* y, int n, int y_rows, const int32_t* dst_row, int num_tokens,
                        uint16_t* out, void* stream) {
  if (n < 0 || y_rows < 0 || num_tokens < 0) return FP8G_EINVAL;
  if (n % 8 != 0) return FP8G_EUNSUPPORTED;
  if (num_tokens == 0 || n == 0) return FP8G_OK;
  if (!dst_row || !out || (y_rows > 0 && !y)) return FP8G_EINVAL;
  if ((y && !aligned(y, 16)) || !aligned(out, 16) || !aligned(dst_row, 4)) return FP8G_EINVAL;
  const unsigned grid = unsigned(cdiv64(num_tokens, 4));
  hipLaunchKernelGGL(fp8g::moe_gather_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), y, n,
                     y_rows, dst_row, num_tokens, out);
  return launched();
}

}  // extern "C"
