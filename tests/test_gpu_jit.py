"""GPU parity of the runtime-specialised GEMMs ("DeepSeek open-source week,
day 3: DeepGEMM", "Core features": kernels compiled at run time per shape):
the default configuration reproduces the ahead-of-time kernels bit for bit
(with and without n and k compiled in), other tile configurations match the
CPU oracle, and a second call finds its kernel loaded."""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_04_amd import binding
from _gpu import (Guarded, assert_close, contiguous_case, dense_case, dev, ld_of, masked_case, require_gpu,
                  run_contiguous, run_dense, run_masked, sa_mn_major, say)

pytestmark = pytest.mark.gpu

D, C, M = binding.FP8G_JIT_DENSE, binding.FP8G_JIT_CONTIGUOUS, binding.FP8G_JIT_MASKED
E4, E5 = binding.FP8G_E4M3, binding.FP8G_E5M2


@pytest.fixture(scope="module", autouse=True)
def fresh_cache(tmp_path_factory):
    prev = binding.fp8_jit_get_cache_dir()
    binding.fp8_jit_set_cache_dir(str(tmp_path_factory.mktemp("jit_cache")))
    yield
    binding.fp8_jit_set_cache_dir(prev)


def run_jit(qa, sa, qb, sb, config=None, a_fmt=E4, b_fmt=E4, workspace=True):
    m, k = qa.shape
    n = qb.shape[0]
    out = Guarded((m, n))
    ws = None
    if workspace:
        c = config if config is not None else binding.fp8_jit_default_config(D, m, n, k)
        nbytes = binding.fp8_jit_gemm_workspace_bytes(m, n, k, c)
        if nbytes:
            ws = torch.empty(nbytes // 4 + 1, dtype=torch.float32, device="cuda")
    binding.fp8_jit_gemm_nt(dev(qa), a_fmt, dev(sa_mn_major(sa)), dev(qb), b_fmt, dev(sb), out.view, config=config,
                            workspace=ws)
    return out.result()


@pytest.mark.parametrize("m,n,k", [(64, 2112, 7168), (128, 4096, 1536), (300, 1000, 2048), (2048, 2048, 512)])
def test_default_config_reproduces_the_ahead_of_time_bits(m, n, k):
    require_gpu()
    say(f"jit default m={m} n={n} k={k}")
    qa, sa, qb, sb = dense_case(m, n, k, seed=k + 1)
    aot = run_dense(qa, sa, qb, sb)
    assert np.array_equal(run_jit(qa, sa, qb, sb), aot)
    spec = binding._config(binding.fp8_jit_default_config(D, m, n, k), specialize=1)
    assert np.array_equal(run_jit(qa, sa, qb, sb, config=spec), aot)
    assert_close(aot, oracle.gemm_nt(qa, sa, qb, sb), f"{m}x{n}x{k}")


TILE_CONFIGS = [
    dict(block_m=64, block_n=64, waves_m=1, waves_n=4, waves_k=1, stages=4, k_per_stage=1, splits=3),
    dict(block_m=128, block_n=128, waves_m=2, waves_n=2, waves_k=1, stages=3, k_per_stage=1, splits=1),
    dict(block_m=256, block_n=128, waves_m=2, waves_n=2, waves_k=1, stages=2, k_per_stage=1, splits=1),
    dict(block_m=64, block_n=32, waves_m=1, waves_n=1, waves_k=4, stages=3, k_per_stage=4, splits=5),
    dict(block_m=128, block_n=64, waves_m=2, waves_n=2, waves_k=2, stages=2, k_per_stage=2, splits=2),
    dict(block_m=64, block_n=128, waves_m=2, waves_n=4, waves_k=1, stages=3, k_per_stage=1, splits=1),
]


@pytest.mark.parametrize("specialize", [0, 1])
@pytest.mark.parametrize("ci", range(len(TILE_CONFIGS)))
def test_tile_configs_match_the_oracle(ci, specialize):
    require_gpu()
    config = dict(TILE_CONFIGS[ci], specialize=specialize)
    assert binding.fp8_jit_config_supported(D, config), config
    m, n, k = 200, 1032, 1664        # tails in M and N, 13 K groups (uneven splits)
    say(f"jit config {ci} specialize={specialize}")
    qa, sa, qb, sb = dense_case(m, n, k, seed=ci)
    got = run_jit(qa, sa, qb, sb, config=config)
    assert_close(got, oracle.gemm_nt(qa, sa, qb, sb), f"config {config}")
    if config["splits"] > 1:        # no workspace: the same tile without splitting
        again = run_jit(qa, sa, qb, sb, config=config, workspace=False)
        assert_close(again, oracle.gemm_nt(qa, sa, qb, sb), "no workspace")


# (split count, k): 13, 14 or 24 K groups, so that each count is one the
# equal runs of K groups actually give
SPLIT_CASES = [(2, 1664), (3, 1664), (4, 1664), (5, 1664), (6, 3072), (7, 1792), (8, 3072)]
SPLIT_TILES = [
    dict(block_m=64, block_n=32, waves_m=4, waves_n=1, waves_k=1, stages=4, k_per_stage=1),    # 2 chunks per thread
    dict(block_m=128, block_n=128, waves_m=4, waves_n=2, waves_k=1, stages=3, k_per_stage=1),  # 8 chunks per thread
]


@pytest.mark.parametrize("ti", range(len(SPLIT_TILES)))
@pytest.mark.parametrize("splits,k", SPLIT_CASES)
def test_every_split_count_matches_the_oracle(splits, k, ti):
    """The last arrival adds 2..8 partials, several chunks per wait when the
    splits are few; tails in M and N leave chunks past the tile's edge."""
    require_gpu()
    m, n = 200, 1032
    config = dict(SPLIT_TILES[ti], splits=splits, specialize=0)
    assert binding.fp8_jit_config_supported(D, config), config
    tiles = -(-m // config["block_m"]) * -(-n // config["block_n"])
    counters = -(-tiles * 8 // 256) * 256
    assert (binding.fp8_jit_gemm_workspace_bytes(m, n, k, config) - counters) // (m * n * 4) == splits
    say(f"jit split-K tile {ti} splits={splits} k={k}")
    qa, sa, qb, sb = dense_case(m, n, k, seed=40 + splits)
    got = run_jit(qa, sa, qb, sb, config=config)
    assert_close(got, oracle.gemm_nt(qa, sa, qb, sb), f"splits={splits} tile {ti}")
    assert np.array_equal(run_jit(qa, sa, qb, sb, config=config), got)


def test_e5m2_specialised():
    require_gpu()
    m, n, k = 96, 4096, 2048
    x, w = np.random.default_rng(4).standard_normal((m, k)).astype(np.float32), \
        np.random.default_rng(5).standard_normal((n, k)).astype(np.float32)
    qa, sa = oracle.cast_1x128(x, fmt=oracle.E5M2)
    qb, sb = oracle.cast_128x128(w, fmt=oracle.E4M3)
    config = binding._config(binding.fp8_jit_default_config(D, m, n, k), specialize=1)
    got = run_jit(qa, sa, qb, sb, config=config, a_fmt=E5, b_fmt=E4)
    assert_close(got, oracle.gemm_nt(qa, sa, qb, sb, a_fmt=oracle.E5M2, b_fmt=oracle.E4M3), "e5m2 x e4m3")


def test_grouped_default_configs_reproduce_the_ahead_of_time_bits():
    require_gpu()
    n, k = 264, 640
    qa, sa, qb, sb, m_idx = contiguous_case([256, 128, 384], n, k, seed=3)
    aot = run_contiguous(qa, sa, qb, sb, m_idx)
    out = Guarded(aot.shape)
    binding.fp8_jit_grouped_gemm_contiguous(dev(qa), dev(sa_mn_major(sa)), dev(qb), dev(sb), out.view,
                                            dev(m_idx.astype(np.int32)))
    assert np.array_equal(out.result(), aot)
    G, max_m = 4, 200
    counts = np.array([0, 200, 77, 129], np.int32)
    qa, sa, qb, sb = masked_case(G, max_m, n, k, counts, seed=4)
    aot = run_masked(qa, sa, qb, sb, counts)
    sa_dev = np.stack([sa_mn_major(sa[g], ld_of(max_m)) for g in range(G)])
    for config in (None, dict(block_m=64, block_n=128, waves_m=1, waves_n=4, waves_k=1, stages=4, k_per_stage=1,
                              splits=1, specialize=1)):
        out = Guarded(aot.shape)
        binding.fp8_jit_grouped_gemm_masked(dev(qa), dev(sa_dev), dev(qb), dev(sb), out.view, dev(counts),
                                            config=config)
        got = out.result()
        for g in range(G):
            assert np.array_equal(got[g, counts[g]:], aot[g, counts[g]:])   # untouched rows keep the sentinel
        if config is None:
            assert np.array_equal(got, aot)
        else:
            for g in range(G):
                c = int(counts[g])
                if c:
                    assert_close(got[g, :c], oracle.gemm_nt(qa[g, :c], sa[g, :c], qb[g], sb[g]), f"group {g}")


def test_second_call_finds_the_kernel_loaded():
    require_gpu()
    m, n, k = 64, 512, 1024
    qa, sa, qb, sb = dense_case(m, n, k, seed=9)
    config = dict(TILE_CONFIGS[1], specialize=1)
    first = run_jit(qa, sa, qb, sb, config=config)
    before = binding.fp8_jit_stats()
    second = run_jit(qa, sa, qb, sb, config=config)
    after = binding.fp8_jit_stats()
    assert after["memory_hits"] == before["memory_hits"] + 1 and after["compiles"] == before["compiles"]
    assert np.array_equal(first, second)


def test_unsupported_config_fails_before_launch():
    require_gpu()
    qa, sa, qb, sb = dense_case(16, 64, 256, seed=1)
    bad = dict(TILE_CONFIGS[0], stages=9)
    with pytest.raises(binding.Fp8GemmError) as e:
        run_jit(qa, sa, qb, sb, config=bad, workspace=False)
    assert e.value.status == binding.FP8G_EUNSUPPORTED


def test_warmed_up_jit_call_replays_in_a_graph():
    """A warmed-up runtime-specialised split-K call captured in a HIP graph and
    replayed several times, with eager work between replays, gives the eager
    bits every time."""
    require_gpu()
    m, n, k = 64, 2048, 4096
    qa, sa, qb, sb = dense_case(m, n, k, seed=13)
    config = dict(TILE_CONFIGS[0], specialize=1)
    binding.fp8_jit_warmup(D, n, k, config=config)
    a, s_, b, t = dev(qa), dev(sa_mn_major(sa)), dev(qb), dev(sb)
    ws = torch.empty(binding.fp8_jit_gemm_workspace_bytes(m, n, k, config) // 4 + 1, dtype=torch.float32,
                     device="cuda")
    eager = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    binding.fp8_jit_gemm_nt(a, E4, s_, b, E4, t, eager, config=config, workspace=ws)
    torch.cuda.synchronize()
    ref = eager.view(torch.int16).cpu().numpy()
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        binding.fp8_jit_gemm_nt(a, E4, s_, b, E4, t, out, config=config, workspace=ws)  # on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        binding.fp8_jit_gemm_nt(a, E4, s_, b, E4, t, out, config=config, workspace=ws)
    for r in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.view(torch.int16).cpu().numpy(), ref), f"replay {r}"
        binding.fp8_jit_gemm_nt(a, E4, s_, b, E4, t, eager, config=config, workspace=ws)   # eager work between
        torch.cuda.synchronize()


def test_cu_limit_slices_give_the_same_bits():
    """A runtime-specialised split-K GEMM under a CU limit (consecutive
    launches of at most that many workgroups) gives the unlimited call's
    bits: the configuration is fixed, and the split partials and arrival
    counts carry across the launches."""
    require_gpu()
    config = dict(TILE_CONFIGS[0], specialize=0)
    qa, sa, qb, sb = dense_case(200, 1032, 1664, seed=11)
    want = run_jit(qa, sa, qb, sb, config=config)
    prev = binding.fp8_set_num_cus(9)
    try:
        say("jit split-K limited to 9 CUs")
        got = run_jit(qa, sa, qb, sb, config=config)
    finally:
        binding.fp8_set_num_cus(prev)
    assert np.array_equal(got, want)



@pytest.mark.parametrize("mode", ["dense_split", "dense_large", "contiguous", "masked"])
def test_single_stage_ring_matches_the_oracle(mode, monkeypatch):
    """The single-buffer debug form (FP8G_PIPELINE_DEPTH=1: one ring stage,
    each stage's copies issued only after every wave has read the last one;
    "DeepGEMM: FP8 GEMM kernel optimisation practice on Hopper Tensor
    Cores", section 6.2) gives results within the bar for every kind."""
    require_gpu()
    monkeypatch.setenv("FP8G_PIPELINE_DEPTH", "1")
    say(f"jit single-stage ring {mode}")
    if mode.startswith("dense"):
        m, n, k = (64, 2112, 7168) if mode == "dense_split" else (512, 520, 1280)
        qa, sa, qb, sb = dense_case(m, n, k, seed=17)
        assert_close(run_jit(qa, sa, qb, sb), oracle.gemm_nt(qa, sa, qb, sb), f"{mode} {m}x{n}x{k}")
    elif mode == "contiguous":
        sizes, n, k = [256, 128, 384], 264, 1024
        qa, sa, qb, sb, m_idx = contiguous_case(sizes, n, k, seed=18)
        out = Guarded((qa.shape[0], n))
        binding.fp8_jit_grouped_gemm_contiguous(dev(qa), dev(sa_mn_major(sa)), dev(qb), dev(sb), out.view,
                                                dev(m_idx.astype(np.int32)))
        ref = np.full((qa.shape[0], n), 0x5A5A, np.uint16)
        oracle.gemm_contiguous(qa, sa, qb, sb, m_idx, ref)
        assert_close(out.result(), ref, "contiguous, one stage")
    else:
        G, max_m, n, k, counts = 3, 128, 264, 1024, [128, 0, 70]
        qa, sa, qb, sb = masked_case(G, max_m, n, k, counts, seed=19)
        out = Guarded((G, max_m, n))
        sa_dev = np.stack([sa_mn_major(sa[g], ld_of(max_m)) for g in range(G)])
        binding.fp8_jit_grouped_gemm_masked(dev(qa), dev(sa_dev), dev(qb), dev(sb), out.view,
                                            dev(np.asarray(counts, np.int32)))
        got = out.result()
        ref = np.full((G, max_m, n), 0x5A5A, np.uint16)
        oracle.gemm_masked(qa, sa, qb, sb, np.asarray(counts, np.int32), ref)
        for g, c in enumerate(counts):
            assert np.all(got[g, c:] == 0x5A5A)
        assert_close(np.concatenate([got[g, :c].ravel() for g, c in enumerate(counts)]),
                     np.concatenate([ref[g, :c].ravel() for g, c in enumerate(counts)]), "masked, one stage")
