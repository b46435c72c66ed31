"""The "Basic usage" call of "DeepSeek open-source week, day 3: DeepGEMM":
m, n, k = 128, 4096, 7168 with both scale tensors filled by randn, so the
scales are signed and of any magnitude (no amax/448 cast in between), and
FP8 codes drawn uniformly over every finite E4M3 value (subnormals, both
zeros and +-448 included).  A promotion that dropped a sign, used |scale|
or mishandled a negative sa * sb would fail here, while every other parity
test's inputs come from the amax/448 casts, whose scales are all positive.

Covered: the dense kind on the page's shape, a split-K shape and the large
256 x 256 tile, and both grouped kinds; every valid output against the
oracle."""
import numpy as np
import pytest

import oracle
from _gpu import (SENTINEL, assert_close, kg_of, require_gpu, run_contiguous, run_dense, run_masked, say)
from fp8_block_scaled_04_amd import binding

pytestmark = pytest.mark.gpu


def uniform_codes(rng, shape):
    """Every finite E4M3FN code with equal probability (0x7F and 0xFF, the
    NaN codes, excluded)."""
    c = rng.integers(0, 254, size=shape, dtype=np.int64)
    c += c >= 0x7F                  # skip 0x7F: 0..0x7E, 0x80..0xFE
    return c.astype(np.uint8)


def randn_scales(rng, shape):
    return rng.standard_normal(shape).astype(np.float32)


@pytest.mark.parametrize("m,n,k", [(128, 4096, 7168),      # the page's example
                                   (64, 2112, 7168),       # 64 x 32 tiles, split-K
                                   (512, 1024, 2048),      # 128 x 64 tiles, split-K
                                   (2048, 4096, 1024)])    # 256 x 256 tiles
def test_dense_signed_randn_scales_uniform_codes(m, n, k):
    require_gpu()
    desc = binding.fp8_gemm_describe(m, n, k)
    say(f"dense signed scales m={m} n={n} k={k} {desc}")
    rng = np.random.default_rng(m + n + k)
    qa, qb = uniform_codes(rng, (m, k)), uniform_codes(rng, (n, k))
    sa, sb = randn_scales(rng, (m, kg_of(k))), randn_scales(rng, ((n + 127) // 128, kg_of(k)))
    assert (sa < 0).any() and (sb < 0).any()
    ref = oracle.gemm_nt(qa, sa, qb, sb)
    got = run_dense(qa, sa, qb, sb)
    assert_close(got, ref, f"{m}x{n}x{k} {desc}")
    if "splits=1 " not in desc:
        assert_close(run_dense(qa, sa, qb, sb, use_workspace=False), ref, f"{m}x{n}x{k} unsplit")


def test_contiguous_signed_randn_scales_uniform_codes():
    require_gpu()
    sizes, n, k = [256, 384, 128], 1024, 7168
    say(f"contiguous signed scales sizes={sizes} n={n} k={k}")
    rng = np.random.default_rng(41)
    M, G, kg, nb = sum(sizes), len(sizes), kg_of(k), (n + 127) // 128
    qa, sa = uniform_codes(rng, (M, k)), randn_scales(rng, (M, kg))
    qb, sb = uniform_codes(rng, (G, n, k)), randn_scales(rng, (G, nb, kg))
    m_idx = np.repeat(np.arange(G, dtype=np.int32), sizes)
    ref = np.full((M, n), SENTINEL, np.uint16)
    oracle.gemm_contiguous(qa, sa, qb, sb, m_idx, ref)
    got = run_contiguous(qa, sa, qb, sb, m_idx)
    assert_close(got, ref, "contiguous, signed scales")


def test_masked_signed_randn_scales_uniform_codes():
    require_gpu()
    G, max_m, n, k = 4, 128, 1024, 7168
    counts = [128, 0, 77, 5]
    say(f"masked signed scales G={G} max_m={max_m} n={n} k={k} counts={counts}")
    rng = np.random.default_rng(43)
    kg, nb = kg_of(k), (n + 127) // 128
    qa, sa = uniform_codes(rng, (G, max_m, k)), randn_scales(rng, (G, max_m, kg))
    qb, sb = uniform_codes(rng, (G, n, k)), randn_scales(rng, (G, nb, kg))
    ref = np.full((G, max_m, n), SENTINEL, np.uint16)
    oracle.gemm_masked(qa, sa, qb, sb, np.asarray(counts, np.int32), ref)
    got = run_masked(qa, sa, qb, sb, counts)
    for g, c in enumerate(counts):
        assert np.all(got[g, c:] == SENTINEL), f"group {g} wrote past its count"
    valid = np.concatenate([got[g, :c].ravel() for g, c in enumerate(counts)])
    want = np.concatenate([ref[g, :c].ravel() for g, c in enumerate(counts)])
    assert_close(valid, want, "masked, signed scales")
