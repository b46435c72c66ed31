"""The Python binding checks every tensor's extent and device against the
sizes the call derives from lhs / rhs, and raises ValueError before the C
library is reached (the C ABI sees raw pointers only, so a short tensor
would otherwise be read or written out of bounds on the device)."""
import pytest
import torch

from fp8_block_scaled_04_amd import binding

pytestmark = pytest.mark.gpu


class _NoLibrary:
    """Stands in for the loaded library: any use of it fails the test."""

    def __getattr__(self, name):
        raise AssertionError(f"the library was called ({name}) although an argument was wrong")


@pytest.fixture
def no_library(monkeypatch):
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    monkeypatch.setattr(binding, "_lib", _NoLibrary())


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8, device="cuda")


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32, device="cuda")


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16, device="cuda")


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32, device="cuda")


M, N, K, G, MAXM = 64, 256, 384, 3, 32     # KG = 3, NB = 2


# (each table entry builds its tensors when its test runs, not at collection)
def dense_args(**bad):
    a = dict(lhs=u8(M, K), lhs_scales=f32(3, M), rhs=u8(N, K), rhs_scales=f32(2, 3), out=bf16(M, N))
    a.update(bad)
    return a


DENSE_BAD = {
    "rhs k differs": lambda: dict(rhs=u8(N, K - 128)),
    "lhs_scales too few rows (ld < m)": lambda: dict(lhs_scales=f32(3, M - 4)),
    "lhs_scales too few K groups": lambda: dict(lhs_scales=f32(2, M)),
    "rhs_scales too few blocks": lambda: dict(rhs_scales=f32(1, 3)),
    "rhs_scales too few K groups": lambda: dict(rhs_scales=f32(2, 2)),
    "out too few rows": lambda: dict(out=bf16(M - 1, N)),
    "out too few columns": lambda: dict(out=bf16(M, N - 8)),
    "lhs not 2-D": lambda: dict(lhs=u8(1, M, K)),
}


@pytest.mark.parametrize("what", sorted(DENSE_BAD))
def test_dense_mismatch_raises_before_the_call(no_library, what):
    a = dense_args(**DENSE_BAD[what]())
    with pytest.raises(ValueError):
        binding.fp8_gemm_nt(a["lhs"], a["lhs_scales"], a["rhs"], a["rhs_scales"], a["out"])
    with pytest.raises(ValueError):
        binding.fp8_gemm_nt_fmt(a["lhs"], binding.FP8G_E4M3, a["lhs_scales"], a["rhs"], binding.FP8G_E5M2,
                                a["rhs_scales"], a["out"])
    with pytest.raises(ValueError):
        binding.fp8_jit_gemm_nt(a["lhs"], binding.FP8G_E4M3, a["lhs_scales"], a["rhs"], binding.FP8G_E4M3,
                                a["rhs_scales"], a["out"])


def test_dense_workspace_on_the_host_raises(no_library):
    a = dense_args()
    with pytest.raises(TypeError):
        binding.fp8_gemm_nt(a["lhs"], a["lhs_scales"], a["rhs"], a["rhs_scales"], a["out"],
                            workspace=torch.zeros(16))


def contiguous_args(**bad):
    a = dict(lhs=u8(M, K), lhs_scales=f32(3, M), rhs=u8(G, N, K), rhs_scales=f32(G, 2, 3), out=bf16(M, N),
             m_indices=i32(M))
    a.update(bad)
    return a


CONTIGUOUS_BAD = {
    "m_indices too short": lambda: dict(m_indices=i32(M - 1)),
    "rhs k differs": lambda: dict(rhs=u8(G, N, K + 128)),
    "rhs_scales for fewer groups": lambda: dict(rhs_scales=f32(G - 1, 2, 3)),
    "lhs_scales ld < m_total": lambda: dict(lhs_scales=f32(3, M - 4)),
    "out too few rows": lambda: dict(out=bf16(M - 8, N)),
    "rhs not 3-D": lambda: dict(rhs=u8(N, K)),
}


@pytest.mark.parametrize("what", sorted(CONTIGUOUS_BAD))
def test_contiguous_mismatch_raises_before_the_call(no_library, what):
    a = contiguous_args(**CONTIGUOUS_BAD[what]())
    for fn in (binding.fp8_grouped_gemm_contiguous, binding.fp8_jit_grouped_gemm_contiguous):
        with pytest.raises(ValueError):
            fn(a["lhs"], a["lhs_scales"], a["rhs"], a["rhs_scales"], a["out"], a["m_indices"])


def masked_args(**bad):
    a = dict(lhs=u8(G, MAXM, K), lhs_scales=f32(G, 3, MAXM), rhs=u8(G, N, K), rhs_scales=f32(G, 2, 3),
             out=bf16(G, MAXM, N), masked_m=i32(G))
    a.update(bad)
    return a


MASKED_BAD = {
    "masked_m too short": lambda: dict(masked_m=i32(G - 1)),
    "rhs for fewer groups": lambda: dict(rhs=u8(G - 1, N, K)),
    "lhs_scales for fewer groups": lambda: dict(lhs_scales=f32(G - 1, 3, MAXM)),
    "lhs_scales ld < max_m": lambda: dict(lhs_scales=f32(G, 3, MAXM - 4)),
    "rhs_scales too few blocks": lambda: dict(rhs_scales=f32(G, 1, 3)),
    "out too few rows": lambda: dict(out=bf16(G, MAXM - 1, N)),
    "lhs not 3-D": lambda: dict(lhs=u8(G * MAXM, K)),
}


@pytest.mark.parametrize("what", sorted(MASKED_BAD))
def test_masked_mismatch_raises_before_the_call(no_library, what):
    a = masked_args(**MASKED_BAD[what]())
    for fn in (binding.fp8_grouped_gemm_masked, binding.fp8_jit_grouped_gemm_masked):
        with pytest.raises(ValueError):
            fn(a["lhs"], a["lhs_scales"], a["rhs"], a["rhs_scales"], a["out"], a["masked_m"])


CAST_BAD = {
    "q too small": lambda: dict(q=u8(M - 1, K)),
    "scales ld < m": lambda: dict(scales=f32(3, M - 4)),
    "scales too few K groups": lambda: dict(scales=f32(2, M)),
}


@pytest.mark.parametrize("what", sorted(CAST_BAD))
def test_cast_mismatch_raises_before_the_call(no_library, what):
    a = dict(x=f32(M, K), q=u8(M, K), scales=f32(3, M))
    a.update(CAST_BAD[what]())
    with pytest.raises(ValueError):
        binding.fp8_cast_per_token_group(a["x"], a["q"], a["scales"])
    with pytest.raises(ValueError):
        binding.fp8_cast_per_token_group_fmt(a["x"], binding.FP8G_E4M3, a["q"], a["scales"])


@pytest.mark.parametrize("what", ["q", "scales"])
def test_block_cast_mismatch_raises_before_the_call(no_library, what):
    a = dict(w=f32(N, K), q=u8(N, K), scales=f32(2, 3))
    a[what] = u8(N, K - 128) if what == "q" else f32(2, 2)
    with pytest.raises(ValueError):
        binding.fp8_cast_per_block(a["w"], a["q"], a["scales"])
    with pytest.raises(ValueError):
        binding.fp8_cast_per_block_fmt(a["w"], binding.FP8G_E5M2, a["q"], a["scales"])


def test_moe_mismatches_raise_before_the_call(no_library):
    T, k, n, kg = 40, 256, 64, 2
    q, s, dst = u8(T, k), f32(kg, T), i32(T)
    with pytest.raises(ValueError):      # dst_row shorter than the tokens
        binding.fp8_moe_scatter_rows(q, s, i32(T - 1), u8(128, k), f32(kg, 128))
    with pytest.raises(ValueError):      # source scales ld < tokens
        binding.fp8_moe_scatter_rows(q, f32(kg, T - 4), dst, u8(128, k), f32(kg, 128))
    with pytest.raises(ValueError):      # laid-out codes of another k
        binding.fp8_moe_scatter_rows(q, s, dst, u8(128, k - 16), f32(kg, 128))
    with pytest.raises(ValueError):      # laid-out scales for fewer groups than the rows span
        binding.fp8_moe_scatter_rows(q, s, dst, u8(4, 32, k), f32(3, kg, 32), rows_per_group=32)
    with pytest.raises(ValueError):      # laid-out scales ld < rows per group
        binding.fp8_moe_scatter_rows(q, s, dst, u8(4, 32, k), f32(4, kg, 28), rows_per_group=32)
    with pytest.raises(ValueError):      # gather output of another token count
        binding.fp8_moe_gather_rows(bf16(128, n), dst, bf16(T + 1, n))
    with pytest.raises(ValueError):      # gather source rows of another width
        binding.fp8_moe_gather_rows(bf16(128, n + 8), dst, bf16(T, n))
    with pytest.raises(ValueError):      # routing given as a matrix
        binding.fp8_moe_layout_masked(i32(4, 10), 4, 16)
