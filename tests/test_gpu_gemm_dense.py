"""GPU parity of the dense block-scaled FP8 NT GEMM against the CPU oracle
("DeepSeek open-source week, day 3: DeepGEMM": "Basic usage" operands and
scales, "Core features" two-level accumulation, BF16 output).

Every output of every workload shape is compared with the oracle, the rms
of the tolerance taken over all of the call's outputs.  Output buffers
carry canary bands, so stray stores fail the test."""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_04_amd import binding
from _gpu import assert_close, dense_case, dev, ld_of, require_gpu, run_dense, sa_mn_major, say, Guarded

pytestmark = pytest.mark.gpu

SMALL_SHAPES = [(1, 8, 128), (16, 64, 256), (63, 136, 384), (64, 2112, 1280), (65, 256, 512),
                (128, 264, 640), (129, 136, 384), (257, 520, 1280), (512, 384, 1024), (300, 1000, 2048)]


@pytest.mark.parametrize("m,n,k", SMALL_SHAPES)
def test_dense_every_output(m, n, k):
    require_gpu()
    say(f"dense every-output m={m} n={n} k={k}")
    qa, sa, qb, sb = dense_case(m, n, k, seed=m + n + k)
    ref = oracle.gemm_nt(qa, sa, qb, sb)
    for ws in (True, False):
        got = run_dense(qa, sa, qb, sb, use_workspace=ws)
        assert_close(got, ref, f"m={m} n={n} k={k} ws={ws}")


# (shape, tile the library picks, split): every m <= 128 tile family, split
# and unsplit, with M and N tails
FAMILY_CASES = [((1, 8, 7168), "64x32", True), ((37, 2112, 1024), "64x32", False),
                ((1, 8200, 128), "64x64", False), ((1, 4096, 12288), "64x64", True),
                ((16, 7168, 12288), "64x64", True), ((65, 7168, 7168), "64x64", False),
                ((1, 16392, 128), "64x128", False), ((1, 8200, 7168), "64x128", True),
                ((65, 8200, 128), "64x128", False), ((65, 16392, 128), "128x128", False),
                ((65, 8200, 7168), "128x128", True)]


@pytest.mark.parametrize("shape,tile,split", FAMILY_CASES)
def test_dense_small_m_tile_families_every_output(shape, tile, split):
    require_gpu()
    m, n, k = shape
    desc = binding.fp8_gemm_describe(m, n, k)
    assert desc.startswith(f"tile={tile} ") and ("splits=1 " not in desc) == split, desc
    say(f"dense family {desc} m={m} n={n} k={k}")
    qa, sa, qb, sb = dense_case(m, n, k, seed=n + k)
    ref = oracle.gemm_nt(qa, sa, qb, sb)
    got = run_dense(qa, sa, qb, sb)
    assert_close(got, ref, f"{m}x{n}x{k} {desc}")
    if split:
        assert np.array_equal(got, run_dense(qa, sa, qb, sb)), "split-K result not deterministic"


@pytest.mark.timeout(300)
def test_dense_k_tail_regression_shape():
    """The K-tail failure shape of the jianying88 practice article (§6.1):
    M = N = 6144, K = 1280, every output."""
    require_gpu()
    m = n = 6144
    k = 1280
    say(f"dense k-tail shape {m}x{n}x{k} (every output)")
    qa, sa, qb, sb = dense_case(m, n, k, seed=61)
    got = run_dense(qa, sa, qb, sb)
    assert_close(got, oracle.gemm_nt(qa, sa, qb, sb), "6144x6144x1280")


def test_dense_config0_full():
    """m=64, n=2112, k=7168, seed 0: every output."""
    require_gpu()
    say("dense m=64 n=2112 k=7168 (every output)")
    qa, sa, qb, sb = dense_case(64, 2112, 7168, seed=0)
    ref = oracle.gemm_nt(qa, sa, qb, sb)
    got = run_dense(qa, sa, qb, sb)
    assert_close(got, ref, "64x2112x7168")
    again = run_dense(qa, sa, qb, sb)
    assert np.array_equal(got, again), "two runs differ"


NK = [(4096, 7168), (7168, 2048), (24576, 1536), (7168, 16384)]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("m", [64, 128, 4096])
@pytest.mark.parametrize("n,k", NK)
def test_dense_config1_sweep(m, n, k):
    """The m x (n, k) sweep, every output."""
    require_gpu()
    say(f"dense sweep m={m} n={n} k={k} (every output)")
    qa, sa, qb, sb = dense_case(m, n, k, seed=0)
    got = run_dense(qa, sa, qb, sb)
    assert_close(got, oracle.gemm_nt(qa, sa, qb, sb), f"{m}x{n}x{k}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("m,n,k", [(8192, 8192, 8192), (16384, 7168, 16384)])
def test_dense_config4_outliers(m, n, k):
    """Large compute-bound shapes with 1% of the elements of both operands
    scaled by 50 before quantisation: every output."""
    require_gpu()
    say(f"dense large m={m} n={n} k={k} (outliers, every output)")
    qa, sa, qb, sb = dense_case(m, n, k, seed=0, outliers=True)
    got = run_dense(qa, sa, qb, sb)
    say(f"  GPU done; oracle over {m * n * k / 1e12:.2f} T MAC")
    assert_close(got, oracle.gemm_nt(qa, sa, qb, sb), f"{m}x{n}x{k}")


def test_dense_split_and_unsplit_agree_and_are_deterministic():
    require_gpu()
    assert "splits=3 " in binding.fp8_gemm_describe(8, 1024, 8192)
    qa, sa, qb, sb = dense_case(8, 1024, 8192, seed=5)
    a = run_dense(qa, sa, qb, sb, use_workspace=True)
    b = run_dense(qa, sa, qb, sb, use_workspace=True)
    c = run_dense(qa, sa, qb, sb, use_workspace=False)
    assert np.array_equal(a, b)
    ref = oracle.gemm_nt(qa, sa, qb, sb)
    assert_close(a, ref, "split")
    assert_close(c, ref, "unsplit")


@pytest.mark.parametrize("m,n,k,cus", [(96, 512, 2048, 16), (64, 2112, 7168, 12), (1024, 2048, 1024, 5),
                                      (300, 1000, 2048, 7)])
def test_dense_cu_limit_does_not_change_results(m, n, k, cus):
    """Under a CU limit the GEMM runs as consecutive launches of at most that
    many workgroups (split-K partials and arrival counts carry across them);
    every output still matches the oracle."""
    require_gpu()
    qa, sa, qb, sb = dense_case(m, n, k, seed=6)
    ref = oracle.gemm_nt(qa, sa, qb, sb)
    prev = binding.fp8_set_num_cus(cus)
    try:
        say(f"dense m={m} n={n} k={k} limited to {cus} CUs: {binding.fp8_gemm_describe(m, n, k)}")
        got = run_dense(qa, sa, qb, sb)
    finally:
        binding.fp8_set_num_cus(prev)
    assert_close(got, ref, f"{cus} CUs")


def test_dense_scale_linearity_on_gpu():
    """Doubling every RHS scale doubles every output exactly (a power-of-two
    scale commutes with every rounding on the way)."""
    require_gpu()
    qa, sa, qb, sb = dense_case(64, 256, 1024, seed=7)
    a = run_dense(qa, sa, qb, sb)
    b = run_dense(qa, sa, qb, sb * np.float32(2.0))
    fa = oracle.bf16_bits_to_f64(a)
    fb = oracle.bf16_bits_to_f64(b)
    assert np.array_equal(fb, 2.0 * fa)


def test_dense_rejects_bad_shapes_before_launch():
    require_gpu()
    lhs = torch.zeros((4, 200), dtype=torch.uint8, device="cuda")
    rhs = torch.zeros((8, 200), dtype=torch.uint8, device="cuda")
    sa = torch.zeros((2, 4), dtype=torch.float32, device="cuda")
    sb = torch.zeros((1, 2), dtype=torch.float32, device="cuda")
    out = Guarded((4, 8))
    with pytest.raises(binding.Fp8GemmError) as e:
        binding.fp8_gemm_nt(lhs, sa, rhs, sb, out.view)
    assert e.value.status == binding.FP8G_EUNSUPPORTED
    res = out.result()
    assert np.all(res == 0x5A5A)
    # misaligned pointer
    lhs2 = torch.zeros((4 * 128 + 8,), dtype=torch.uint8, device="cuda")[8:].view(4, 128)
    with pytest.raises(binding.Fp8GemmError) as e:
        binding.fp8_gemm_nt(lhs2, sa[:1], rhs[:, :128].contiguous(), sb[:, :1].contiguous(), out.view)
    assert e.value.status == binding.FP8G_EINVAL


def test_dense_zero_rows_is_a_noop():
    require_gpu()
    lhs = torch.zeros((0, 128), dtype=torch.uint8, device="cuda")
    rhs = torch.zeros((8, 128), dtype=torch.uint8, device="cuda")
    sa = torch.zeros((1, 4), dtype=torch.float32, device="cuda")
    sb = torch.zeros((1, 1), dtype=torch.float32, device="cuda")
    out = torch.empty((0, 8), dtype=torch.bfloat16, device="cuda")
    binding.fp8_gemm_nt(lhs, sa, rhs, sb, out)
    torch.cuda.synchronize()


def _dense_dev(qa, sa, qb, sb):
    from _gpu import sa_mn_major
    return dev(qa), dev(sa_mn_major(sa)), dev(qb), dev(sb)


@pytest.mark.parametrize("m,n,k", [(8, 1024, 8192), (128, 512, 7168)])
def test_splitk_workspace_needs_no_initialisation(m, n, k):
    """The split-K arrival counters carry a tag: a workspace full of
    random bytes gives the same bits as a zeroed one, call after call."""
    require_gpu()
    qa, sa, qb, sb = dense_case(m, n, k, seed=11)
    a, s_, b, t = _dense_dev(qa, sa, qb, sb)
    nbytes = binding.fp8_gemm_workspace_bytes(m, n, k)
    assert nbytes > 0, "shape expected to use split-K"
    ws0 = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
    junk = np.random.default_rng(3).integers(0, 256, nbytes, dtype=np.uint8)
    ws1 = dev(junk).view(torch.float32)
    outs = []
    for ws in (ws0, ws1, ws1, ws0):
        out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        binding.fp8_gemm_nt(a, s_, b, t, out, workspace=ws)
        outs.append(out.view(torch.int16).cpu().numpy().view(np.uint16))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    assert_close(outs[0], oracle.gemm_nt(qa, sa, qb, sb), "split-K")


def test_splitk_workspace_shared_by_shapes_in_turn():
    """Split shapes with different tile grids and split counts take turns on
    one workspace, so each one's counter words sit where another left
    partial sums or counts: every call gives the bits of the same call on a
    workspace of its own."""
    require_gpu()
    shapes = [(64, 2048, 7168), (128, 512, 7168), (8, 1024, 8192), (64, 4096, 7168)]
    cases, refs = [], []
    for i, (m, n, k) in enumerate(shapes):
        desc = binding.fp8_gemm_describe(m, n, k)
        say(f"dense {m}x{n}x{k}: {desc}")
        assert "splits=1 " not in desc, desc
        qa, sa, qb, sb = dense_case(m, n, k, seed=20 + i)
        args = _dense_dev(qa, sa, qb, sb)
        own = torch.zeros(binding.fp8_gemm_workspace_bytes(m, n, k) // 4, dtype=torch.float32, device="cuda")
        out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        binding.fp8_gemm_nt(*args, out, workspace=own)
        torch.cuda.synchronize()
        cases.append((m, n, args))
        refs.append(out.view(torch.int16).cpu().numpy())
        if i == 0:
            assert_close(refs[0].view(np.uint16), oracle.gemm_nt(qa, sa, qb, sb), "split-K, own workspace")
    nbytes = max(binding.fp8_gemm_workspace_bytes(m, n, k) for m, n, k in shapes)
    shared = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
    for i in [0, 1, 2, 3, 3, 0, 2, 1, 0, 0, 3, 2]:
        m, n, args = cases[i]
        out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        binding.fp8_gemm_nt(*args, out, workspace=shared)
        torch.cuda.synchronize()
        assert np.array_equal(out.view(torch.int16).cpu().numpy(), refs[i]), f"shape {shapes[i]}"


def test_splitk_graph_replay_matches_eager():
    """A captured split-K call, replayed several times with eager work in
    between, reproduces the eager result bit for bit each time."""
    require_gpu()
    m, n, k = 64, 2048, 7168
    assert "splits=1 " not in binding.fp8_gemm_describe(m, n, k)
    qa, sa, qb, sb = dense_case(m, n, k, seed=12)
    a, s_, b, t = _dense_dev(qa, sa, qb, sb)
    ws = torch.zeros(binding.fp8_gemm_workspace_bytes(m, n, k) // 4, dtype=torch.float32, device="cuda")
    eager = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    binding.fp8_gemm_nt(a, s_, b, t, eager, workspace=ws)
    torch.cuda.synchronize()
    ref = eager.view(torch.int16).cpu().numpy()
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        binding.fp8_gemm_nt(a, s_, b, t, out, workspace=ws)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        binding.fp8_gemm_nt(a, s_, b, t, out, workspace=ws)
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.view(torch.int16).cpu().numpy(), ref), f"replay {rep}"
        # eager work on the same workspace between replays
        binding.fp8_gemm_nt(a, s_, b, t, eager, workspace=ws)
        torch.cuda.synchronize()


def test_cu_limit_slices_replay_in_a_graph():
    """Under a CU limit a GEMM is several launches; captured into a HIP graph
    and replayed with eager work in between, they reproduce the eager
    result bit for bit (split-K partials and arrival counts included)."""
    require_gpu()
    m, n, k = 256, 512, 7168         # 128x64 tiles, 2 splits, 32 workgroups in slices of 24
    qa, sa, qb, sb = dense_case(m, n, k, seed=13)
    a, s_, b, t = _dense_dev(qa, sa, qb, sb)
    prev = binding.fp8_set_num_cus(24)
    try:
        desc = binding.fp8_gemm_describe(m, n, k)
        say(f"dense {m}x{n}x{k} limited to 24 CUs: {desc}")
        grid = int(desc.split("grid=")[1])
        assert grid > 24 and "splits=1 " not in desc, desc   # more than one slice, split-K
        ws = torch.zeros(binding.fp8_gemm_workspace_bytes(m, n, k) // 4 + 1, dtype=torch.float32, device="cuda")
        eager = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        binding.fp8_gemm_nt(a, s_, b, t, eager, workspace=ws)
        torch.cuda.synchronize()
        ref = eager.view(torch.int16).cpu().numpy()
        out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            binding.fp8_gemm_nt(a, s_, b, t, out, workspace=ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            binding.fp8_gemm_nt(a, s_, b, t, out, workspace=ws)
        for rep in range(3):
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(out.view(torch.int16).cpu().numpy(), ref), f"replay {rep}"
            binding.fp8_gemm_nt(a, s_, b, t, eager, workspace=ws)
            torch.cuda.synchronize()
    finally:
        binding.fp8_set_num_cus(prev)
    assert_close(ref.view(np.uint16), oracle.gemm_nt(qa, sa, qb, sb), "24 CUs, graph")


@pytest.mark.parametrize("m,n,k", [(16, 264, 65536), (200, 136, 65536)])
def test_dense_maximum_k(m, n, k):
    """k = 65536, the largest the kernels take (512 K groups, every RHS scale
    row of a tile held in LDS): split and unsplit paths against the oracle."""
    require_gpu()
    say(f"dense maximum k m={m} n={n} k={k} {binding.fp8_gemm_describe(m, n, k)}")
    qa, sa, qb, sb = dense_case(m, n, k, seed=7)
    ref = oracle.gemm_nt(qa, sa, qb, sb)
    for ws in (True, False):
        assert_close(run_dense(qa, sa, qb, sb, use_workspace=ws), ref, f"{m}x{n}x{k} ws={ws}")


def test_dense_maximum_k_256_tile():
    """The 256 x 256 tile (through the runtime specialisation, one tile) at k = 65536."""
    require_gpu()
    m, n, k = 256, 256, 65536
    qa, sa, qb, sb = dense_case(m, n, k, seed=8)
    config = dict(block_m=256, block_n=256, waves_m=4, waves_n=2, waves_k=1, stages=2, k_per_stage=1, splits=1,
                  specialize=0)
    out = Guarded((m, n))
    binding.fp8_jit_gemm_nt(dev(qa), binding.FP8G_E4M3, dev(sa_mn_major(sa)), dev(qb), binding.FP8G_E4M3, dev(sb),
                            out.view, config=config)
    assert_close(out.result(), oracle.gemm_nt(qa, sa, qb, sb), "256x256x65536")


def _device_codes(rows, k, seed):
    """Seeded random E4M3 codes made on the device (an operand this large is
    slow to make on the host): uniform over every finite code, NaN (0x7f,
    0xff) excluded."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    c = torch.randint(0, 254, (rows, k), dtype=torch.uint8, device="cuda", generator=g)
    c += (c >= 127).to(torch.uint8)
    return c


@pytest.mark.timeout(300)
@pytest.mark.parametrize("side", ["lhs", "rhs"])
def test_dense_operand_past_4gib(side):
    """An operand of more than 4 GiB (266,240 rows of k = 16384), LHS or RHS:
    every output against the oracle, so rows (LHS) or columns (RHS) on both
    sides of the first 4 GiB are covered."""
    require_gpu()
    big, small, k = 266240, (256 if side == "lhs" else 64), 16384
    m, n = (big, small) if side == "lhs" else (small, big)
    say(f"dense operand past 4 GiB side={side} m={m} n={n} k={k} {binding.fp8_gemm_describe(m, n, k)}")
    kg, g = k // 128, torch.Generator(device="cuda").manual_seed(11)
    a = _device_codes(m, k, seed=12)
    b = _device_codes(n, k, seed=13)
    sa = (0.5 + torch.rand(kg, ld_of(m), device="cuda", generator=g)) * 1e-2     # MN-major
    sb = (0.5 + torch.rand((n + 127) // 128, kg, device="cuda", generator=g)) * 1e-2
    out = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    nbytes = binding.fp8_gemm_workspace_bytes(m, n, k)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda") if nbytes else None
    binding.fp8_gemm_nt(a, sa, b, sb, out, workspace=ws)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    qa, qb = a.cpu().numpy(), b.cpu().numpy()
    del a, b
    sa_rows, sb_h = sa[:, :m].T.contiguous().cpu().numpy(), sb.cpu().numpy()
    say(f"  GPU done; oracle over {m * n * k / 1e12:.2f} T MAC")
    assert_close(got, oracle.gemm_nt(qa, sa_rows, qb, sb_h), f"{side} past 4 GiB")
