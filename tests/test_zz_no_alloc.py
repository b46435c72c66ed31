"""fp8_gemm_nt_noalloc, the entry point for callers that cannot allocate:
its split-K scratch is the library's static per-device array.  Called
through the C ABI, it must reproduce fp8_gemm_nt (with a workspace) bit for
bit, on two calls in a row (the second smaller, so the array holds the
first call's counters and partials), in a HIP graph replayed with eager
calls in between, and refuse before launching a problem whose split-K
scratch would not fit."""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_04_amd import binding
from _gpu import Guarded, assert_close, dense_case, dev, require_gpu, run_dense, sa_mn_major, say

pytestmark = pytest.mark.gpu


def _noalloc(qa, sa, qb, sb):
    m, n = qa.shape[0], qb.shape[0]
    out = Guarded((m, n))
    binding.fp8_gemm_nt_noalloc(dev(qa), dev(sa_mn_major(sa)), dev(qb), dev(sb), out.view)
    return out.result()


def test_noalloc_matches_the_workspace_entry_point_twice_in_a_row():
    require_gpu()
    for (m, n, k), seed in [((64, 7168, 16384), 31), ((8, 1024, 8192), 32)]:   # the second is smaller
        desc = binding.fp8_gemm_describe(m, n, k)
        assert "splits=1 " not in desc, desc            # both use the split-K scratch
        say(f"no-allocation GEMM m={m} n={n} k={k} {desc}")
        qa, sa, qb, sb = dense_case(m, n, k, seed=seed)
        got = _noalloc(qa, sa, qb, sb)
        want = run_dense(qa, sa, qb, sb, use_workspace=True)
        assert np.array_equal(got, want), f"{m}x{n}x{k}: differs from fp8_gemm_nt"
        assert_close(got, oracle.gemm_nt(qa, sa, qb, sb), f"{m}x{n}x{k}")


def test_noalloc_replays_in_a_graph():
    """Captured and replayed with eager calls of another shape in between
    (which rewrite the shared array): every replay gives the eager bits."""
    require_gpu()
    m, n, k = 64, 2112, 7168
    qa, sa, qb, sb = dense_case(m, n, k, seed=33)
    a, s_, b, t = dev(qa), dev(sa_mn_major(sa)), dev(qb), dev(sb)
    q2, s2, b2, t2 = dense_case(8, 1024, 8192, seed=34)
    a2, sa2, bb2, tt2 = dev(q2), dev(sa_mn_major(s2)), dev(b2), dev(t2)
    other = torch.empty((8, 1024), dtype=torch.bfloat16, device="cuda")
    eager = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    binding.fp8_gemm_nt_noalloc(a, s_, b, t, eager)
    torch.cuda.synchronize()
    ref = eager.view(torch.int16).cpu().numpy()
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        binding.fp8_gemm_nt_noalloc(a, s_, b, t, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.fp8_gemm_nt_noalloc(a, s_, b, t, out)
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.view(torch.int16).cpu().numpy(), ref), f"replay {rep}"
        binding.fp8_gemm_nt_noalloc(a2, sa2, bb2, tt2, other)
        torch.cuda.synchronize()
    assert_close(ref.view(np.uint16), oracle.gemm_nt(qa, sa, qb, sb), "graph")


def test_noalloc_refuses_a_problem_whose_scratch_does_not_fit(monkeypatch):
    """Eight splits forced on a 128 x 32768 output need 128 MiB of partial
    sums: refused with FP8G_ESCRATCH, nothing written."""
    require_gpu()
    monkeypatch.setenv("FP8G_SPLITS", "8")
    m, n, k = 128, 32768, 1024
    assert "splits=8 " in binding.fp8_gemm_describe(m, n, k)
    a = torch.zeros((m, k), dtype=torch.uint8, device="cuda")
    s_ = torch.ones((k // 128, m), dtype=torch.float32, device="cuda")
    b = torch.zeros((n, k), dtype=torch.uint8, device="cuda")
    t = torch.ones((n // 128, k // 128), dtype=torch.float32, device="cuda")
    out = Guarded((m, n))
    with pytest.raises(binding.Fp8GemmError) as e:
        binding.fp8_gemm_nt_noalloc(a, s_, b, t, out.view)
    assert e.value.status == binding.FP8G_ESCRATCH
    assert np.all(out.result() == 0x5A5A)
