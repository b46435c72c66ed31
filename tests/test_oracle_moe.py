"""Pins of the MoE layout oracle (oracle/moe.py) against a hand-computed
example and against independent formulations (a stable library sort, exact
integer invariants)."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "moe_layout_small.txt")


def _golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = [int(v) for v in rest]
    return vals


def test_golden_example():
    g = _golden()
    G = g["num_groups"][0]
    counts, offsets, dst, m_idx = oracle.moe_layout_contiguous(g["expert_idx"], G, g["m_rows"][0],
                                                               align=g["align"][0])
    assert counts.tolist() == g["counts"]
    assert offsets.tolist() == g["offsets"]
    assert dst.tolist() == g["dst_contiguous"]
    assert m_idx.tolist() == g["m_indices"]
    counts2, dst2, mm = oracle.moe_layout_masked(g["expert_idx"], G, g["max_m"][0])
    assert counts2.tolist() == g["counts"]
    assert dst2.tolist() == g["dst_masked"]
    assert mm.tolist() == g["masked_m"]


def _routing(seed, T, G, unrouted=0.05):
    rng = np.random.default_rng(seed)
    e = rng.integers(0, G, T)
    bad = rng.random(T) < unrouted
    e[bad] = rng.choice([-1, G, G + 7], bad.sum())
    if G > 3:
        e[e == 1] = 0  # an empty expert
    return e.astype(np.int32)


@pytest.mark.parametrize("T,G", [(1, 1), (17, 3), (1000, 8), (5000, 64), (3000, 300)])
def test_contiguous_matches_stable_sort(T, G):
    """dst_row equals the position a stable library sort gives each token
    inside its expert's block; the layout's invariants hold exactly."""
    e = _routing(T + G, T, G)
    m_rows = oracle.moe_contiguous_rows(T, G)
    counts, offsets, dst, m_idx = oracle.moe_layout_contiguous(e, G, m_rows)
    valid = (e >= 0) & (e < G)
    assert np.array_equal(counts, np.bincount(e[valid], minlength=G))
    assert offsets[0] == 0 and np.all(offsets % 128 == 0)
    assert np.array_equal(np.diff(offsets), (counts + 127) // 128 * 128)
    assert offsets[-1] <= m_rows
    # independent formulation: stable argsort of the routed tokens
    order = np.argsort(np.where(valid, e, G), kind="stable")
    first = np.concatenate([[0], np.cumsum(counts)])
    expect = np.full(T, -1)
    for pos, t in enumerate(order[:valid.sum()]):
        g = e[t]
        expect[t] = offsets[g] + (pos - first[g])
    assert np.array_equal(dst, expect)
    # every routed token lands on a distinct row of its own expert
    assert np.all(dst[~valid] == -1)
    assert len(set(dst[valid].tolist())) == valid.sum()
    assert np.array_equal(m_idx[dst[valid]], e[valid])
    assert np.all(m_idx[offsets[-1]:] == -1)


@pytest.mark.parametrize("T,G,max_m", [(50, 4, 8), (2000, 16, 256), (700, 5, 1)])
def test_masked_keeps_first_tokens(T, G, max_m):
    e = _routing(T * 3 + G, T, G)
    counts, dst, mm = oracle.moe_layout_masked(e, G, max_m)
    assert np.array_equal(mm, np.minimum(counts, max_m))
    valid = (e >= 0) & (e < G)
    for g in range(G):
        toks = np.nonzero(e == g)[0]
        kept = toks[:max_m]
        assert np.array_equal(dst[kept], g * max_m + np.arange(kept.size))
        assert np.all(dst[toks[max_m:]] == -1)
    assert np.all(dst[~valid] == -1)


def test_scatter_then_gather_is_identity():
    rng = np.random.default_rng(5)
    T, G, k, n = 300, 6, 256, 64
    e = _routing(9, T, G)
    m_rows = oracle.moe_contiguous_rows(T, G)
    _, _, dst, _ = oracle.moe_layout_contiguous(e, G, m_rows)
    q = rng.integers(0, 256, (T, k), dtype=np.uint8)
    s = rng.random((T, 2)).astype(np.float32)
    q_out = np.zeros((m_rows, k), np.uint8)
    s_out = np.zeros((m_rows, 2), np.float32)
    oracle.moe_scatter_rows(q, s, dst, m_rows, m_rows, q_out, s_out)
    routed = dst >= 0
    assert np.array_equal(q_out[dst[routed]], q[routed])
    assert np.array_equal(s_out[dst[routed]], s[routed])
    y = rng.integers(0, 65536, (m_rows, n), dtype=np.uint16)
    back = oracle.moe_gather_rows(y, dst, n)
    assert np.array_equal(back[routed], y[dst[routed]])
    assert np.all(back[~routed] == 0)
