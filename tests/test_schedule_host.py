"""The tile scheduler, checked on the host (no device): for random shapes,
random contiguous group indices (runs of odd and even length, skipped
blocks, groups interleaved block by block, more blocks than a wave has
lanes), random masked counts (negative, zero, past max_m, more groups than a
wave has lanes), split-K and CU limits that cut a call into consecutive
launches, every work unit that has work is taken by exactly one workgroup,
and no workgroup takes anything else.

fp8_gemm_schedule decodes each workgroup with the functions the kernels
run (the XCD share, the dense tile order, the contiguous run scan and tile
lookup, the masked live-unit numbering) through the same launch slicing as
the GEMM entry points.  The expected units are computed here, in plain
numpy, from the layouts' definitions ("DeepSeek open-source week, day 3:
DeepGEMM": a contiguous layout's rows carry their group, a masked layout's
groups their valid-row counts)."""
import os

import numpy as np
import pytest

from fp8_block_scaled_04_amd import binding, build

DENSE, CONTIGUOUS, MASKED = binding.FP8G_JIT_DENSE, binding.FP8G_JIT_CONTIGUOUS, binding.FP8G_JIT_MASKED
CASES = 4000          # per kind: 12,000 random cases in all


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(build.LIB):
        build.build()
    binding.lib()
    if binding.fp8_get_num_cus() != 256:
        pytest.skip("the configurations checked are those of a 256-CU device (or no device)")
    yield
    binding.fp8_set_num_cus(0)


def cu_limit(rng):
    """No limit half the time, else a limit that slices most grids."""
    return 0 if rng.random() < 0.5 else int(rng.integers(1, 300))


def as_sorted(rows):
    a = np.asarray(rows, np.int64).reshape(-1, 5)
    return a[np.lexsort(a.T[::-1])]


def check(units, expected, what):
    taken = units[units[:, 0] == 1][:, 1:]
    idle = units[units[:, 0] == 0]
    assert np.all(np.isin(units[:, 0], (0, 1))), what
    assert np.all(idle[:, 1] == -1), f"{what}: a workgroup found no lane holding its tile"
    got = as_sorted(taken)
    want = as_sorted(expected)
    assert got.shape == want.shape, f"{what}: {got.shape[0]} units taken, {want.shape[0]} expected"
    assert np.array_equal(got, want), f"{what}: the units taken differ from the expected ones"


def test_dense_every_tile_and_split_exactly_once(lib):
    rng = np.random.default_rng(2024)
    for case in range(CASES):
        lim = cu_limit(rng)
        binding.fp8_set_num_cus(lim)
        if rng.random() < 0.5:
            m = int(rng.integers(1, 129))                    # the small-M families, split-K
        else:
            m = int(rng.integers(129, 3000))
        n = 8 * int(rng.integers(1, 700))
        k = 128 * int(rng.integers(1, 80))
        desc = binding.fp8_gemm_describe(m, n, k)
        tile = desc.split()[0][5:].split("x")
        bm, bn = int(tile[0]), int(tile[1])
        splits = int(desc.split("splits=")[1].split()[0])
        units = binding.fp8_gemm_schedule(DENSE, m, n, k)
        tm, tn = -(-m // bm), -(-n // bn)
        assert units.shape[0] == tm * tn * splits, desc
        i, j, s = np.meshgrid(np.arange(tm), np.arange(tn), np.arange(splits), indexing="ij")
        i, j, s = i.ravel(), j.ravel(), s.ravel()
        exp = np.stack([np.zeros_like(i), i * bm, np.minimum(bm, m - i * bm), j, s], 1)
        check(units, exp, f"dense case {case} m={m} n={n} k={k} limit={lim} {desc}")
    binding.fp8_set_num_cus(0)


def random_blocks(rng):
    """Group index of each 128-row block: runs of random groups and
    lengths, skipped blocks (-1), or groups alternating block by block."""
    nblk = int(rng.integers(1, 200))
    G = int(rng.integers(1, 12))
    style = rng.integers(0, 3)
    if style == 0:            # runs of random length, some skipped
        out = []
        while len(out) < nblk:
            out += [int(rng.integers(-1, G))] * int(rng.integers(1, 8))
        return np.array(out[:nblk], np.int32), G
    if style == 1:            # interleaved block by block
        return rng.integers(-1, G, nblk).astype(np.int32), G
    # experts in order, each a whole number of blocks (the usual layout), then padding
    sizes = rng.integers(0, 10, G)
    out = np.repeat(np.arange(G, dtype=np.int32), sizes)
    return np.concatenate([out, np.full(int(rng.integers(0, 4)), -1, np.int32)]), G


def contiguous_tiles(blocks):
    """Each maximal run of equal non-negative indices cut into tiles of two
    blocks from its first block (an odd run ends in a one-block tile)."""
    tiles = []
    b = 0
    while b < len(blocks):
        e = b
        while e < len(blocks) and blocks[e] == blocks[b]:
            e += 1
        if blocks[b] >= 0:
            for t in range(b, e, 2):
                tiles.append((int(blocks[b]), 128 * t, 128 * min(2, e - t)))
        b = e
    return tiles


def test_contiguous_every_tile_exactly_once(lib):
    rng = np.random.default_rng(7)
    for case in range(CASES):
        lim = cu_limit(rng)
        binding.fp8_set_num_cus(lim)
        blocks, G = random_blocks(rng)
        if blocks.size == 0:
            continue
        m_indices = np.repeat(blocks, 128)
        M = m_indices.size
        n = 8 * int(rng.integers(1, 200))
        units = binding.fp8_gemm_schedule(CONTIGUOUS, M, n, 256, G, m_indices)
        tn = -(-n // 256)
        assert units.shape[0] == (M // 128) * tn
        exp = [(g, r0, rows, j, 0) for (g, r0, rows) in contiguous_tiles(blocks) for j in range(tn)]
        check(units, exp, f"contiguous case {case} blocks={blocks.tolist()} n={n} limit={lim}")
    binding.fp8_set_num_cus(0)


def test_masked_every_live_unit_exactly_once(lib):
    rng = np.random.default_rng(11)
    tile = binding.fp8_jit_default_config(MASKED, 1, 1024, 128)  # the masked kernel's tile
    bm, bn = tile.block_m, tile.block_n
    for case in range(CASES):
        lim = cu_limit(rng)
        binding.fp8_set_num_cus(lim)
        G = int(rng.integers(1, 100))
        max_m = int(rng.integers(1, 400))
        counts = rng.integers(-5, max_m + 20, G).astype(np.int32)
        counts[rng.random(G) < 0.3] = 0
        n = 8 * int(rng.integers(1, 160))
        units = binding.fp8_gemm_schedule(MASKED, max_m, n, 128, G, counts)
        tn = -(-n // bn)
        assert units.shape[0] == -(-max_m // bm) * tn * G
        exp = []
        for g in range(G):
            rows = min(max(int(counts[g]), 0), max_m)
            for i in range(-(-rows // bm)):
                for j in range(tn):
                    exp.append((g, i * bm, min(bm, rows - i * bm), j, 0))
        check(units, exp, f"masked case {case} G={G} max_m={max_m} counts={counts.tolist()} n={n} limit={lim}")
    binding.fp8_set_num_cus(0)


def test_schedule_rejects_what_the_gemms_reject(lib):
    lib_ = binding.lib()
    assert lib_.fp8_gemm_schedule(DENSE, 64, 8, 100, 0, None, None, 0) == binding.FP8G_EUNSUPPORTED
    assert lib_.fp8_gemm_schedule(CONTIGUOUS, 100, 8, 128, 2, None, None, 0) == binding.FP8G_EUNSUPPORTED
    assert lib_.fp8_gemm_schedule(MASKED, 64, 8, 128, 2, None, None, 0) == binding.FP8G_EINVAL
    assert lib_.fp8_gemm_schedule(7, 64, 8, 128, 0, None, None, 0) == binding.FP8G_EINVAL
    assert lib_.fp8_gemm_schedule(DENSE, 0, 8, 128, 0, None, None, 0) == 0
