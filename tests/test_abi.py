"""CPU-only checks of the C-ABI library: it loads, exports every function
include/fp8gemm.h declares, and rejects bad arguments on the host before any
launch.  No call here reaches a kernel."""
import ctypes
import os
import re

import pytest

from fp8_block_scaled_04_amd import binding, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(build.LIB):
        build.build()
    return binding.lib()


def test_exports_every_declared_function(lib):
    names = binding.header_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(binding._SIGNATURES)


def test_status_strings(lib):
    assert binding.status_string(0) == "ok"
    assert "invalid" in binding.status_string(-1)
    assert "unsupported" in binding.status_string(-2)
    assert "launch" in binding.status_string(-3)
    assert "unknown" in binding.status_string(7)


def test_host_validation_paths(lib):
    g = lib.fp8_gemm_nt
    # null pointers
    assert g(None, None, 4, None, None, None, 4, 8, 128, None, 0, None) == binding.FP8G_EINVAL
    # negative sizes
    assert g(None, None, 4, None, None, None, -1, 8, 128, None, 0, None) == binding.FP8G_EINVAL
    # K not a multiple of 128, N not a multiple of 8, K too large
    assert g(None, None, 4, None, None, None, 4, 8, 100, None, 0, None) == binding.FP8G_EUNSUPPORTED
    assert g(None, None, 4, None, None, None, 4, 12, 128, None, 0, None) == binding.FP8G_EUNSUPPORTED
    assert g(None, None, 4, None, None, None, 4, 8, 128 * 513, None, 0, None) == binding.FP8G_EUNSUPPORTED
    # zero-sized problems are no-ops
    assert g(None, None, 4, None, None, None, 0, 8, 128, None, 0, None) == binding.FP8G_OK
    assert g(None, None, 4, None, None, None, 4, 0, 128, None, 0, None) == binding.FP8G_OK
    c = lib.fp8_grouped_gemm_contiguous
    assert c(None, None, 128, None, None, None, None, 100, 8, 128, 2, None, 0, None) == binding.FP8G_EUNSUPPORTED
    assert c(None, None, 128, None, None, None, None, 128, 8, 128, 2, None, 0, None) == binding.FP8G_EINVAL
    assert c(None, None, 128, None, None, None, None, 0, 8, 128, 2, None, 0, None) == binding.FP8G_OK
    mk = lib.fp8_grouped_gemm_masked
    assert mk(None, None, 4, None, None, None, None, 2, 4, 8, 128, None, 0, None) == binding.FP8G_EINVAL
    assert mk(None, None, 4, None, None, None, None, 0, 4, 8, 128, None, 0, None) == binding.FP8G_OK
    assert mk(None, None, 4, None, None, None, None, -1, 4, 8, 128, None, 0, None) == binding.FP8G_EINVAL
    t = lib.fp8_cast_per_token_group
    assert t(None, 0, 4, 128, None, None, 4, None) == binding.FP8G_EINVAL
    assert t(None, 5, 4, 128, None, None, 4, None) == binding.FP8G_EINVAL
    assert t(None, 0, 4, 12, None, None, 4, None) == binding.FP8G_EUNSUPPORTED
    b = lib.fp8_cast_per_block
    assert b(None, 4, 128, None, None, None) == binding.FP8G_EINVAL
    assert b(None, 4, 6, None, None, None) == binding.FP8G_EUNSUPPORTED


def test_scale_leading_dimension_limits(lib):
    """ld below the rows, not a multiple of 4, or past 32 bits is refused
    before anything is launched (the pointers are placeholders that are
    never dereferenced: with no device present a launch could not happen
    anyway, and with one this test does not run)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("placeholder pointers are only passed where no device exists")
    p = ctypes.c_void_p(1 << 20)
    g = lib.fp8_gemm_nt
    for ld in (4, 6, 2 ** 31, 2 ** 32 + 8):
        assert g(p, p, ld, p, p, p, 8, 8, 128, None, 0, None) == binding.FP8G_EUNSUPPORTED, ld
    mk = lib.fp8_grouped_gemm_masked
    assert mk(p, p, 2 ** 31 + 4, p, p, p, p, 2, 8, 8, 128, None, 0, None) == binding.FP8G_EUNSUPPORTED
    c = lib.fp8_grouped_gemm_contiguous
    assert c(p, p, 2 ** 31, p, p, p, p, 128, 8, 128, 2, None, 0, None) == binding.FP8G_EUNSUPPORTED


def test_describe_reports_the_tile_choice(lib):
    """Host-only tile choice for a 256-CU device: 256 x 256 tiles for large
    M, narrow split tiles for small M."""
    if binding.fp8_get_num_cus() != 256:
        pytest.skip("the expectations are for a 256-CU device (or no device)")
    d = binding.fp8_gemm_describe
    for shape in [(4096, 7168, 16384), (4096, 4096, 7168), (4096, 24576, 1536), (8192, 8192, 8192)]:
        assert d(*shape).startswith("tile=256x256 "), shape
    assert "splits=1 grid=448" in d(4096, 7168, 16384)
    small = d(64, 2112, 7168)
    assert small.startswith("tile=64x32 ") and "splits=1" not in small
    assert d(0, 8, 128) == "empty"
    with pytest.raises(binding.Fp8GemmError):
        d(4, 8, 100)
    buf = ctypes.create_string_buffer(8)
    assert lib.fp8_gemm_describe(4096, 7168, 16384, buf, 8) == binding.FP8G_OK
    assert buf.value == b"tile=25"        # truncated, NUL-terminated
    assert lib.fp8_gemm_describe(4, 8, 128, None, 8) == binding.FP8G_EINVAL
    assert lib.fp8_gemm_describe(-1, 8, 128, buf, 8) == binding.FP8G_EINVAL


def test_format_entry_points_validate(lib):
    E4, E5 = binding.FP8G_E4M3, binding.FP8G_E5M2
    g = lib.fp8_gemm_nt_fmt
    for fa, fb in ((2, E4), (E4, -1), (E5, 7)):
        assert g(None, fa, None, 4, None, fb, None, None, 4, 8, 128, None, 0, None) == binding.FP8G_EINVAL
    for fa, fb in ((E4, E4), (E5, E4), (E4, E5), (E5, E5)):
        # the same size checks as the E4M3 entry point, and empty problems are no-ops
        assert g(None, fa, None, 4, None, fb, None, None, 4, 8, 100, None, 0, None) == binding.FP8G_EUNSUPPORTED
        assert g(None, fa, None, 4, None, fb, None, None, 0, 8, 128, None, 0, None) == binding.FP8G_OK
    t = lib.fp8_cast_per_token_group_fmt
    assert t(None, 0, 3, 0, 128, None, None, 4, None) == binding.FP8G_EINVAL
    assert t(None, 0, E5, 4, 128, None, None, 4, None) == binding.FP8G_EINVAL
    assert t(None, 0, E5, 4, 12, None, None, 4, None) == binding.FP8G_EUNSUPPORTED
    b = lib.fp8_cast_per_block_fmt
    assert b(None, 2, 0, 128, None, None, None) == binding.FP8G_EINVAL
    assert b(None, E5, 4, 6, None, None, None) == binding.FP8G_EUNSUPPORTED
    with pytest.raises(ValueError):
        binding._fmt(2, "q_format")


def test_cu_limit_setter(lib):
    prev = binding.fp8_set_num_cus(17)
    try:
        assert binding.fp8_set_num_cus(3) == 17
        assert 1 <= binding.fp8_get_num_cus() <= 3
    finally:
        binding.fp8_set_num_cus(prev)


def test_oracle_and_gpu_path_share_nothing():
    """The oracle is test infrastructure: the package never imports it, it
    never imports the package, and no source file is shared."""
    pkg = os.path.join(ROOT, "fp8_block_scaled_04_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "fp8_oracle" not in text, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".cpp")):
            text = open(os.path.join(ROOT, "oracle", f)).read()
            assert "fp8_block_scaled_04_amd" not in text, f
            assert "fp8gemm" not in text and "hip" not in text.lower().replace("ship", ""), f


def test_split_override_only_where_split_k_can_run(lib, monkeypatch):
    """FP8G_SPLITS (a tuning override) changes the split count only where
    split-K is possible: never for the 256 x 256 tile, whose ring cannot
    stage a split partial, and never without a workspace."""
    if binding.fp8_get_num_cus() != 256:
        pytest.skip("the expectations are for a 256-CU device (or no device)")
    monkeypatch.setenv("FP8G_SPLITS", "4")
    d = binding.fp8_gemm_describe
    for shape in [(4096, 7168, 16384), (8192, 8192, 8192)]:
        desc = d(*shape)
        assert desc.startswith("tile=256x256 ") and "splits=1 " in desc, desc
        assert binding.fp8_gemm_workspace_bytes(*shape) == 0
    assert "splits=4 " in d(64, 2112, 7168)          # the override itself works where split-K runs
    assert binding.fp8_gemm_workspace_bytes(64, 2112, 7168) > 0


def test_noalloc_entry_point_host_checks(lib):
    """fp8_gemm_nt_noalloc checks its arguments like fp8_gemm_nt, before it
    looks up its scratch or launches anything."""
    g = lib.fp8_gemm_nt_noalloc
    assert g(None, None, 4, None, None, None, 4, 8, 128, None) == binding.FP8G_EINVAL
    assert g(None, None, 4, None, None, None, -1, 8, 128, None) == binding.FP8G_EINVAL
    assert g(None, None, 4, None, None, None, 4, 8, 100, None) == binding.FP8G_EUNSUPPORTED
    assert g(None, None, 4, None, None, None, 0, 8, 128, None) == binding.FP8G_OK
    assert "scratch" in binding.status_string(binding.FP8G_ESCRATCH)
