"""Block-scaled FP8 GEMM for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libfp8gemm.so`` (hand-written HIP
kernels, built by :mod:`fp8_block_scaled_04_amd.build`); :mod:`.binding`
exposes its entry points under the same names.  :mod:`.synth` generates the
seeded synthetic inputs used by the tests and the benchmark.
"""
from .binding import (  # noqa: F401
    FP8G_BF16, FP8G_E4M3, FP8G_E5M2, FP8G_EINVAL, FP8G_ELAUNCH, FP8G_EUNSUPPORTED, FP8G_F32, FP8G_OK,
    Fp8GemmError, fp8_cast_per_block, fp8_cast_per_block_fmt, fp8_cast_per_token_group,
    fp8_cast_per_token_group_fmt, fp8_gemm_describe, fp8_gemm_nt, fp8_gemm_nt_fmt,
    fp8_gemm_workspace_bytes, fp8_get_num_cus, fp8_grouped_gemm_contiguous,
    fp8_grouped_gemm_masked, fp8_set_num_cus, fp8_status_string,
    fp8_moe_contiguous_rows, fp8_moe_gather_rows, fp8_moe_layout_contiguous, fp8_moe_layout_masked,
    fp8_moe_layout_workspace_bytes, fp8_moe_scatter_rows,
    FP8G_JIT_CONTIGUOUS, FP8G_JIT_DENSE, FP8G_JIT_MASKED, Fp8GemmConfig, fp8_jit_config_supported,
    fp8_jit_default_config, fp8_jit_gemm_nt, fp8_jit_gemm_workspace_bytes, fp8_jit_get_cache_dir,
    fp8_jit_grouped_gemm_contiguous, fp8_jit_grouped_gemm_masked, fp8_jit_set_cache_dir, fp8_jit_stats,
    fp8_jit_warmup,
)
