// Launches of the dense GEMM kernels, one object file per operand-format
// pair (dense_launch.hip is compiled once for each FMT value), so that the
// library's instantiations build in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gemm_kernel.hpp"

namespace fp8g {
namespace host {

// Launches the kernel of dense configuration `kind` (a DenseKind) with
// operand formats FMT (bit 0: LHS E5M2, bit 1: RHS E5M2), split-K or not.
// Returns FP8G_OK, or FP8G_EUNSUPPORTED (launching nothing) for a (kind,
// split) pair that has no kernel.
template <int FMT>
int launch_dense_kind(bool split, int kind, const GemmParams& p, int64_t grid, hipStream_t s);

extern template int launch_dense_kind<0>(bool, int, const GemmParams&, int64_t, hipStream_t);
extern template int launch_dense_kind<1>(bool, int, const GemmParams&, int64_t, hipStream_t);
extern template int launch_dense_kind<2>(bool, int, const GemmParams&, int64_t, hipStream_t);
extern template int launch_dense_kind<3>(bool, int, const GemmParams&, int64_t, hipStream_t);

}  // namespace host
}  // namespace fp8g
