// Dense GEMM instantiations for one operand-format pair, FP8G_DENSE_FMT
// (0..3; the build compiles this file once per value).  Every instantiation
// matches its row of kShapes: tile, wave grid, ring depth, K groups per
// stage and waves sharing a sub-tile.
#include "dense_launch.hpp"
#include "host_common.hpp"

#ifndef FP8G_DENSE_FMT
#define FP8G_DENSE_FMT 0
#endif

namespace fp8g {
namespace host {
namespace {

template <int BM, int BN, int WMW, int WNW, int ST, bool SPLIT, int KU, int WK, int FMT>
void launch(const GemmParams& p, int64_t grid, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WMW, WNW, ST, kDense, SPLIT, KU, WK, FMT>), dim3(unsigned(grid)),
                     dim3(64 * WMW * WNW * WK), 0, s, p);
}

template <bool SPLIT, int FMT>
int launch_kind(int kind, const GemmParams& p, int64_t grid, hipStream_t s) {
  switch (kind) {
    case kS128N64: launch<128, 64, 2, 2, 4, SPLIT, 1, 1, FMT>(p, grid, s); return FP8G_OK;
    case kF64N32: launch<64, 32, 4, 1, 4, SPLIT, 2, 1, FMT>(p, grid, s); return FP8G_OK;
    case kF64N64: launch<64, 64, 2, 2, 4, SPLIT, 2, 2, FMT>(p, grid, s); return FP8G_OK;
    case kF64N128: launch<64, 128, 4, 2, 4, SPLIT, 1, 1, FMT>(p, grid, s); return FP8G_OK;
    case kF128N128: launch<128, 128, 4, 2, 3, SPLIT, 1, 1, FMT>(p, grid, s); return FP8G_OK;
    case kBig:
      // the 256 x 256 tile cannot stage a split partial in its ring
      if constexpr (SPLIT) return FP8G_EUNSUPPORTED;
      else { launch<256, 256, 4, 2, 2, false, 1, 1, FMT>(p, grid, s); return FP8G_OK; }
    default: return FP8G_EUNSUPPORTED;
  }
}

}  // namespace

template <int FMT>
int launch_dense_kind(bool split, int kind, const GemmParams& p, int64_t grid, hipStream_t s) {
  return split ? launch_kind<true, FMT>(kind, p, grid, s) : launch_kind<false, FMT>(kind, p, grid, s);
}

template int launch_dense_kind<FP8G_DENSE_FMT>(bool, int, const GemmParams&, int64_t, hipStream_t);

}  // namespace host
}  // namespace fp8g
