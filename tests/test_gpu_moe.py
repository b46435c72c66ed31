"""GPU parity of the MoE layout steps (the kwkr.cn DeepGEMM usage article,
section 3.2 and the section 4.3 flow: sort tokens by expert, count, grouped
GEMM, restore token order) against the CPU oracle: layouts, counts and row
moves bit for bit; the whole prefill and decode flows within the GEMM
tolerance."""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_04_amd import binding, synth
from _gpu import SENTINEL, assert_close, dev, kg_of, ld_of, require_gpu, say

pytestmark = pytest.mark.gpu


def routing(seed, T, G, unrouted=0.03, empty=True):
    """Expert index per token: uniform over experts, a few tokens routed
    nowhere (-1 or past the last expert), expert 1 left empty."""
    u = synth.uniform(seed, synth.S_GROUP_SIZES, 2 * T)
    e = np.minimum((u[:T] * G).astype(np.int64), G - 1)
    bad = u[T:] < unrouted
    e[bad] = np.where(np.arange(T)[bad] % 2 == 0, -1, G + 2)
    if empty and G > 3:
        e[e == 1] = 0
    return e.astype(np.int32)


# up to 4096 tokens one workgroup does the whole layout (experts matched by
# ballot up to 64 experts, by lane shuffles above); past that, three passes
@pytest.mark.parametrize("T,G", [(1, 1), (1023, 8), (1024, 8), (1025, 64), (4000, 200), (4096, 8), (4097, 8),
                                 (16384, 8), (20000, 256), (70000, 1024)])
def test_layout_contiguous_matches_oracle(T, G):
    require_gpu()
    say(f"moe layout contiguous T={T} G={G}")
    e = routing(T + G, T, G)
    m_rows = binding.fp8_moe_contiguous_rows(T, G)
    assert m_rows == oracle.moe_contiguous_rows(T, G)
    ws = torch.full((binding.fp8_moe_layout_workspace_bytes(T, G) // 4 + 1,), 0x7B7B7B7B, dtype=torch.int32,
                    device="cuda")  # garbage: the workspace needs no initialisation
    counts, offsets, dst, m_idx = binding.fp8_moe_layout_contiguous(dev(e), G, m_rows, workspace=ws)
    rc, ro, rd, rm = oracle.moe_layout_contiguous(e, G, m_rows)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(dst.cpu().numpy(), rd)
    assert np.array_equal(m_idx.cpu().numpy(), rm)


@pytest.mark.parametrize("T,G,max_m", [(1, 1, 1), (300, 16, 8), (2048, 16, 256), (5000, 16, 256), (3000, 1000, 4),
                                       (4096, 64, 300), (4097, 16, 2000), (16384, 64, 300)])
def test_layout_masked_matches_oracle(T, G, max_m):
    require_gpu()
    say(f"moe layout masked T={T} G={G} max_m={max_m}")
    e = routing(T * 7 + G, T, G)
    counts, dst, mm = binding.fp8_moe_layout_masked(dev(e), G, max_m)
    rc, rd, rm = oracle.moe_layout_masked(e, G, max_m)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(dst.cpu().numpy(), rd)
    assert np.array_equal(mm.cpu().numpy(), rm)


def test_layout_rejects_too_few_rows():
    require_gpu()
    e = dev(np.zeros(10, np.int32))
    with pytest.raises(binding.Fp8GemmError) as err:
        binding.fp8_moe_layout_contiguous(e, 4, m_rows=binding.fp8_moe_contiguous_rows(10, 4) - 128)
    assert err.value.status == binding.FP8G_EINVAL


# k = 8320: 65 K groups (several scale chunks per token, a partial last one)
# and 520 16-byte pieces per row; n = 4160: 520 pieces per output row (more
# than one batch of loads per lane in both copies)
@pytest.mark.parametrize("k,n", [(384, 72), (8320, 4160)])
@pytest.mark.parametrize("layout", ["contiguous", "masked"])
def test_scatter_and_gather_bit_exact(layout, k, n):
    require_gpu()
    say(f"moe scatter/gather {layout} k={k} n={n}")
    rng = np.random.default_rng(3)
    T, G = 777, 6
    kg = kg_of(k)
    e = routing(11, T, G)
    q = rng.integers(0, 256, (T, k), dtype=np.uint8)
    s_log = rng.random((T, kg)).astype(np.float32)
    s_dev = np.zeros((kg, ld_of(T)), np.float32)
    s_dev[:, :T] = s_log.T
    if layout == "contiguous":
        rows = binding.fp8_moe_contiguous_rows(T, G)
        _, _, dst, _ = oracle.moe_layout_contiguous(e, G, rows)
        rpg, ld_out = rows, ld_of(rows)
        q_out = torch.full((rows, k), 0xEE, dtype=torch.uint8, device="cuda")
        s_out = torch.full((kg, ld_out), -3.0, dtype=torch.float32, device="cuda")
    else:
        max_m = 100
        rows = G * max_m
        _, dst, _ = oracle.moe_layout_masked(e, G, max_m)
        rpg, ld_out = max_m, ld_of(max_m)
        q_out = torch.full((G, max_m, k), 0xEE, dtype=torch.uint8, device="cuda")
        s_out = torch.full((G, kg, ld_out), -3.0, dtype=torch.float32, device="cuda")
    binding.fp8_moe_scatter_rows(dev(q), dev(s_dev), dev(dst), q_out, s_out, rows_per_group=rpg)
    ref_q = np.full((rows, k), 0xEE, np.uint8)
    ref_s = np.full((rows, kg), -3.0, np.float32)
    oracle.moe_scatter_rows(q, s_log, dst, rows, rpg, ref_q, ref_s)
    got_q = q_out.cpu().numpy().reshape(rows, k)
    assert np.array_equal(got_q, ref_q)
    if layout == "contiguous":
        got_s = s_out.cpu().numpy()[:, :rows].T
    else:
        got_s = s_out.cpu().numpy()[:, :, :max_m].transpose(0, 2, 1).reshape(rows, kg)
    assert np.array_equal(got_s.view(np.uint32), ref_s.view(np.uint32))
    # back to token order
    y = rng.integers(0, 65536, (rows, n), dtype=np.uint16)
    out = torch.full((T, n), 0x1234, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    binding.fp8_moe_gather_rows(dev(y.view(np.int16)).view(torch.bfloat16), dev(dst), out)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.moe_gather_rows(y, dst, n))


def _experts(G, n, k, seed):
    w = synth.normal_f32(seed, synth.S_RHS, (G, n, k))
    qb = np.empty((G, n, k), np.uint8)
    sb = np.empty((G, (n + 127) // 128, kg_of(k)), np.float32)
    for g in range(G):
        qb[g], sb[g] = oracle.cast_128x128(w[g])
    return qb, sb


def _reference(qa, sa, qb, sb, e, n, kept):
    """Token t's output row: its quantised activations times its expert's
    weights (the oracle's dense GEMM, one expert at a time); zeros for
    tokens that are not computed."""
    T = qa.shape[0]
    ref = np.zeros((T, n), np.uint16)
    for g in range(qb.shape[0]):
        toks = np.nonzero(kept & (e == g))[0]
        if toks.size:
            ref[toks] = oracle.gemm_nt(qa[toks], sa[toks], qb[g], sb[g])
    return ref


def test_prefill_flow_end_to_end():
    """x -> per-token-group cast -> contiguous layout -> row scatter ->
    contiguous grouped GEMM -> gather back to token order."""
    require_gpu()
    T, G, k, n = 900, 5, 512, 264
    say(f"moe prefill flow T={T} G={G} k={k} n={n}")
    e = routing(21, T, G)
    x = synth.normal_f32(21, synth.S_LHS, (T, k))
    qb, sb = _experts(G, n, k, 21)
    kg = kg_of(k)
    # GPU path
    xq = torch.empty((T, k), dtype=torch.uint8, device="cuda")
    xs = torch.empty((kg, ld_of(T)), dtype=torch.float32, device="cuda")
    binding.fp8_cast_per_token_group(dev(x), xq, xs)
    rows = binding.fp8_moe_contiguous_rows(T, G)
    _, _, dst, m_idx = binding.fp8_moe_layout_contiguous(dev(e), G, rows)
    q_lay = torch.zeros((rows, k), dtype=torch.uint8, device="cuda")
    s_lay = torch.zeros((kg, ld_of(rows)), dtype=torch.float32, device="cuda")
    binding.fp8_moe_scatter_rows(xq, xs, dst, q_lay, s_lay)
    y = torch.empty((rows, n), dtype=torch.bfloat16, device="cuda")
    binding.fp8_grouped_gemm_contiguous(q_lay, s_lay, dev(qb), dev(sb), y, m_idx)
    out = torch.full((T, n), 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    binding.fp8_moe_gather_rows(y, dst, out)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    # oracle path (its own cast of the same x)
    qa, sa = oracle.cast_1x128(x)
    routed = (e >= 0) & (e < G)
    ref = _reference(qa, sa, qb, sb, e, n, routed)
    assert_close(got[routed], ref[routed], "prefill flow")
    assert np.all(got[~routed] == 0)


def test_decode_flow_end_to_end():
    """x -> cast -> masked layout (a slot of max_m rows per expert, overflow
    dropped) -> scatter -> masked grouped GEMM -> gather."""
    require_gpu()
    T, G, max_m, k, n = 400, 4, 96, 384, 136
    say(f"moe decode flow T={T} G={G} max_m={max_m}")
    e = routing(33, T, G, empty=False)
    x = synth.normal_f32(33, synth.S_LHS, (T, k))
    qb, sb = _experts(G, n, k, 33)
    kg = kg_of(k)
    xq = torch.empty((T, k), dtype=torch.uint8, device="cuda")
    xs = torch.empty((kg, ld_of(T)), dtype=torch.float32, device="cuda")
    binding.fp8_cast_per_token_group(dev(x), xq, xs)
    _, dst, mm = binding.fp8_moe_layout_masked(dev(e), G, max_m)
    q_lay = torch.zeros((G, max_m, k), dtype=torch.uint8, device="cuda")
    s_lay = torch.zeros((G, kg, ld_of(max_m)), dtype=torch.float32, device="cuda")
    binding.fp8_moe_scatter_rows(xq, xs, dst, q_lay, s_lay, rows_per_group=max_m)
    y = torch.full((G, max_m, n), 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    binding.fp8_grouped_gemm_masked(q_lay, s_lay, dev(qb), dev(sb), y, mm)
    out = torch.full((T, n), 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    binding.fp8_moe_gather_rows(y.view(G * max_m, n), dst, out)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    qa, sa = oracle.cast_1x128(x)
    _, rdst, _ = oracle.moe_layout_masked(e, G, max_m)
    kept = rdst >= 0
    assert (~kept & (e >= 0) & (e < G)).any(), "the case should drop some tokens"
    ref = _reference(qa, sa, qb, sb, e, n, kept)
    assert_close(got[kept], ref[kept], "decode flow")
    assert np.all(got[~kept] == 0)
