"""Pins for the CPU oracle: every check compares it with something other than
itself -- closed forms the pages print, torch's own float8_e4m3fn and
bfloat16 conversions, exact integer or rational recomputation, brute force on
tiny inputs, and numpy's float64 matmul.

Sources: "DeepSeek open-source week, day 3: DeepGEMM" (explinks.com),
"Basic usage" and "Source walk-through" part 3; the dpshk.com GEMM/FP8 essay
§3.1 and §3.3; the kwkr.cn DeepGEMM usage article §3.1 and §4.2.
"""
import bisect
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_04_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---- independent helpers (library routines and exhaustive searches) -------
def torch_e4m3_values(codes):
    """Values of E4M3FN codes as torch decodes them (float64)."""
    t = torch.tensor(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_e4m3_encode(x):
    """torch's float32 -> float8_e4m3fn conversion (round to nearest even)."""
    t = torch.tensor(np.asarray(x, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


_BF16_POS = None


def _bf16_positive_table():
    """All positive finite bf16 values as exact Fractions, sorted, with bits."""
    global _BF16_POS
    if _BF16_POS is None:
        bits = np.arange(0x0000, 0x7F80, dtype=np.uint32)
        vals = (bits << 16).view(np.float32)
        _BF16_POS = ([Fraction(float(v)) for v in vals], [int(b) for b in bits])
    return _BF16_POS


def bf16_nearest_exact(q: Fraction) -> int:
    """Nearest bf16 to the exact rational q, ties to the even bit pattern,
    by search of the full table (overflow past the last finite value's
    rounding range gives inf)."""
    vals, bits = _bf16_positive_table()
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    top = vals[-1]
    ulp_top = top - vals[-2]
    if a >= top + ulp_top / 2:
        return sign | 0x7F80
    i = bisect.bisect_left(vals, a)
    if i < len(vals) and vals[i] == a:
        return sign | bits[i]
    lo, hi = i - 1, i
    if hi >= len(vals):
        return sign | bits[lo]
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick = hi if (dhi < dlo or (dhi == dlo and bits[hi] % 2 == 0)) else lo
    return sign | bits[pick]


def e4m3_exact(code) -> Fraction:
    return Fraction(float(torch_e4m3_values([code])[0]))


def rand_finite_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    bad = (c & 0x7F) == 0x7F
    c[bad] = 0x7E & c[bad] | (c[bad] & 0x80)
    return c


# ---- golden facts the pages print -----------------------------------------
def test_golden_format_facts():
    """E4M3 max about 448 and min normal about 2^-6 (dpshk essay §3.1, the
    jianying88 practice article's §3.1 format table); the day-3 page's usage
    example: m,n,k = 128,4096,7168 with scales [m][ceil(k/128)] and
    [ceil(n/128)][ceil(k/128)]."""
    facts = {}
    with open(os.path.join(GOLDEN, "pages_facts.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                key, val = line.split("=", 1)
                facts[key.strip()] = val.strip()
    t = oracle.e4m3_table()
    assert t[0x7E] == float(facts["e4m3_max"])
    assert np.nanmax(t) == float(facts["e4m3_max"])
    assert t[0x08] == 2.0 ** int(facts["e4m3_min_normal_log2"])
    m, n, k = (int(v) for v in facts["usage_mnk"].split(","))
    x = synth.normal_f32(0, 1, (m, k))
    w = synth.normal_f32(0, 2, (n, k))
    _, sa = oracle.cast_1x128(x)
    _, sb = oracle.cast_128x128(w)
    assert sa.shape == tuple(int(v) for v in facts["usage_lhs_scales_shape"].split(","))
    assert sb.shape == tuple(int(v) for v in facts["usage_rhs_scales_shape"].split(","))


# ---- P1: decode table --------------------------------------------------------
def test_p1_decode_table_closed_forms():
    t = oracle.e4m3_table()
    nan = np.isnan(t)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert t[0x7E] == 448.0 and t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9
    assert t[0x38] == 1.0 and t[0x00] == 0.0
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])


def test_p1_decode_table_matches_torch():
    t = oracle.e4m3_table()
    ref = torch_e4m3_values(np.arange(256, dtype=np.uint8))
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(t), ~fin)
    assert np.array_equal(t[fin], ref[fin])
    assert np.array_equal(np.signbit(t[fin]), np.signbit(ref[fin]))


# ---- P2: encoder ---------------------------------------------------------------
def test_p2_roundtrip_every_finite_code():
    t = oracle.e4m3_table()
    codes = np.array([c for c in range(256) if not np.isnan(t[c])], np.uint8)
    assert np.array_equal(oracle.e4m3_encode(t[codes]), codes)


def test_p2_midpoints_go_to_even_code():
    t = oracle.e4m3_table()
    for c in range(0, 0x7E):
        mid = (t[c] + t[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode([mid])[0] == want, hex(c)
        assert oracle.e4m3_encode([-mid])[0] == (0x80 | want), hex(c)


def test_p2_saturation_and_nan():
    q = oracle.e4m3_encode([448.0, 463.9, 464.0, 500.0, 1e30, np.inf, -448.5, -np.inf, np.nan])
    assert list(q[:6]) == [0x7E] * 6
    assert list(q[6:8]) == [0xFE, 0xFE]
    assert q[8] == 0x7F


def test_p2_encoder_matches_torch_and_bruteforce():
    rng = np.random.default_rng(1)
    t = oracle.e4m3_table()
    # random magnitudes over the whole range, plus points just around each
    # midpoint and each code
    x = np.concatenate([
        rng.standard_normal(20000) * 40,
        np.exp(rng.uniform(np.log(1e-5), np.log(447.0), 20000)) * rng.choice([-1, 1], 20000),
    ]).astype(np.float32)
    mids = ((t[:0x7E] + t[1:0x7F]) / 2).astype(np.float32)
    near = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1000)),
                           np.nextafter(t[:0x7F].astype(np.float32), np.float32(1000))])
    x = np.concatenate([x, near, -near, mids, -mids]).astype(np.float32)
    ours = oracle.e4m3_encode(x.astype(np.float64))
    assert np.array_equal(ours, torch_e4m3_encode(x))
    # exhaustive nearest search on a subsample, written independently
    fin = [(Fraction(float(t[c])), c) for c in range(0x7F)]
    for idx in range(0, x.size, 97):
        v = x[idx]
        a = Fraction(float(abs(v)))
        best = min(fin, key=lambda p: (abs(p[0] - a), p[1] % 2))
        want = best[1] | (0x80 if np.signbit(v) else 0)
        assert ours[idx] == want, (float(v), hex(ours[idx]), hex(want))


# ---- bf16 rounding -------------------------------------------------------------
def test_bf16_rne_matches_torch_on_floats():
    rng = np.random.default_rng(2)
    with np.errstate(over="ignore", invalid="ignore"):
        x = np.concatenate([rng.standard_normal(50000) * 10.0 ** rng.integers(-40, 38, 50000),
                            (np.arange(0, 1 << 16, dtype=np.uint32) << 16 | 0x8000).view(np.float32)])
        x = x.astype(np.float32)
    x = x[np.isfinite(x)]
    ours = oracle.bf16_rne(x.astype(np.float64))
    ref = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_rne_from_double_is_single_rounding():
    """Doubles just past a bf16 midpoint must round away from it (rounding
    through fp32 first would land on the midpoint and then tie to even)."""
    one = Fraction(1)
    cases = [1 + 2.0 ** -8 + 2.0 ** -30, 1 + 2.0 ** -8 - 2.0 ** -30, 1 + 2.0 ** -8,
             1 + 3 * 2.0 ** -8, 3.0e38, 3.3961e38, 3.4e38, 1e-39, 2.0 ** -134, 2.0 ** -133 * 1.5,
             -(1 + 2.0 ** -8 + 2.0 ** -40), 0.0, -0.0]
    rng = np.random.default_rng(3)
    cases += list(rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000))
    ours = oracle.bf16_rne(np.array(cases, np.float64))
    for v, o in zip(cases, ours):
        want = bf16_nearest_exact(Fraction(v)) if v != 0 else (0x8000 if np.signbit(v) else 0)
        assert o == want, (v, hex(o), hex(want))
    assert oracle.bf16_rne([np.nan])[0] & 0x7FFF > 0x7F80
    assert list(oracle.bf16_rne([np.inf, -np.inf])) == [0x7F80, 0xFF80]
    del one


# ---- P3: exact group sums -------------------------------------------------------
def test_p3_group_sums_exact_against_int64():
    rng = np.random.default_rng(4)
    m, n, k = 6, 9, 128
    A = rand_finite_codes(rng, (m, k))
    B = rand_finite_codes(rng, (n, k))
    ones_a = np.ones((m, 1), np.float32)
    ones_b = np.ones((1, 1), np.float32)
    _, pre = oracle.gemm_nt(A, ones_a, B, ones_b, want_pre=True)
    ma = (torch_e4m3_values(A) * 512).astype(np.int64)   # integer mantissas
    mb = (torch_e4m3_values(B) * 512).astype(np.int64)
    exact = ma @ mb.T                                      # units of 2^-18
    assert np.array_equal(pre * 2.0 ** 18, exact.astype(np.float64))
    assert np.all(np.abs(exact) < 2 ** 43)


# ---- P4: one-hot and identity ---------------------------------------------------
def test_p4_one_hot_identity_exact():
    m, n, k = 7, 200, 384          # 3 K groups, 2 N blocks (second partial)
    kg, nb = 3, 2
    rng = np.random.default_rng(5)
    pos = rng.integers(0, k, size=m)
    A = np.zeros((m, k), np.uint8)
    A[np.arange(m), pos] = 0x38                       # 1.0
    perm = rng.permutation(k)[:n]                     # B row j is one-hot at perm[j]
    B = np.zeros((n, k), np.uint8)
    B[np.arange(n), perm] = 0x38
    B[0, :] = 0
    B[0, pos[0]] = 0x38                               # force a hit for row 0
    sa = (2.0 ** rng.integers(-6, 6, size=(m, kg))).astype(np.float32)
    sb = (2.0 ** rng.integers(-6, 6, size=(nb, kg))).astype(np.float32)
    out = oracle.gemm_nt(A, sa, B, sb)
    want = np.zeros((m, n), np.float64)
    for i in range(m):
        for j in range(n):
            if B[j, pos[i]] == 0x38:
                g = pos[i] // 128
                want[i, j] = sa[i, g] * sb[j // 128, g]
    assert out[0, 0] != 0
    assert np.array_equal(out, oracle.bf16_rne(want))
    ref = torch.tensor(want.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, ref)


# ---- P5: small integers ---------------------------------------------------------
def test_p5_small_integers_exact():
    rng = np.random.default_rng(6)
    m, n, k = 5, 260, 300          # partial K group and partial N block
    kg, nb = 3, 3
    ints = np.arange(-8, 9)
    codes = torch_e4m3_encode(ints.astype(np.float32))
    ia = rng.integers(0, ints.size, size=(m, k))
    ib = rng.integers(0, ints.size, size=(n, k))
    A, B = codes[ia], codes[ib]
    va, vb = ints[ia].astype(np.int64), ints[ib].astype(np.int64)
    ea = rng.integers(-4, 4, size=(m, kg))
    eb = rng.integers(-4, 4, size=(nb, kg))
    sa = (2.0 ** ea).astype(np.float32)
    sb = (2.0 ** eb).astype(np.float32)
    out, pre = oracle.gemm_nt(A, sa, B, sb, want_pre=True)
    for i in range(m):
        for j in range(n):
            tot = Fraction(0)
            for g in range(kg):
                sl = slice(128 * g, min(128 * g + 128, k))
                dot = int(va[i, sl] @ vb[j, sl])
                tot += Fraction(dot) * Fraction(2) ** int(ea[i, g] + eb[j // 128, g])
            assert Fraction(pre[i, j]) == tot
            assert out[i, j] == bf16_nearest_exact(tot)


# ---- P6: scale linearity --------------------------------------------------------
def test_p6_scale_linearity():
    rng = np.random.default_rng(7)
    m, n, k = 8, 140, 256
    A = rand_finite_codes(rng, (m, k))
    B = rand_finite_codes(rng, (n, k))
    sa = rng.uniform(0.5, 2.0, size=(m, 2)).astype(np.float32)
    sb = rng.uniform(-2.0, 2.0, size=(2, 2)).astype(np.float32)
    out, pre = oracle.gemm_nt(A, sa, B, sb, want_pre=True)
    out2, pre2 = oracle.gemm_nt(A, sa * np.float32(8.0), B, sb, want_pre=True)
    assert np.array_equal(pre2, pre * 8.0)
    bits = out.astype(np.int32)
    nz = (bits & 0x7FFF) != 0
    assert np.array_equal(out2.astype(np.int32)[nz], bits[nz] + (3 << 7))
    out3, pre3 = oracle.gemm_nt(A, sa, B, sb * np.float32(0.25), want_pre=True)
    assert np.array_equal(pre3, pre * 0.25)
    # perturb one LHS scale: only that row moves, by delta * sb * S_g
    sa4 = sa.copy()
    sa4[3, 1] += np.float32(0.5)
    _, pre4 = oracle.gemm_nt(A, sa4, B, sb, want_pre=True)
    diff = pre4 - pre
    assert np.all(diff[np.arange(m) != 3] == 0)
    ones_a = np.zeros((m, 2), np.float32); ones_a[:, 1] = 1
    _, s1 = oracle.gemm_nt(A, ones_a, B, np.ones((2, 2), np.float32), want_pre=True)
    want = (float(sa4[3, 1]) - float(sa[3, 1])) * sb[np.arange(n) // 128, 1].astype(np.float64) * s1[3]
    np.testing.assert_allclose(diff[3], want, rtol=1e-12, atol=1e-9 * np.abs(pre).max())
    # uniform scales reduce to per-tensor scaling
    _, pu = oracle.gemm_nt(A, np.full((m, 2), 0.5, np.float32), B, np.full((2, 2), 4.0, np.float32), want_pre=True)
    va, vb = torch_e4m3_values(A), torch_e4m3_values(B)
    assert np.array_equal(pu, (va @ vb.T) * 2.0)


# ---- P7: brute force on tiny inputs ----------------------------------------------
def test_p7_bruteforce_rational():
    rng = np.random.default_rng(8)
    m, n, k = 3, 131, 259            # partial last K group and N block
    kg, nb = 3, 2
    A = rand_finite_codes(rng, (m, k))
    B = rand_finite_codes(rng, (n, k))
    sa = rng.standard_normal((m, kg)).astype(np.float32)
    sb = rng.standard_normal((nb, kg)).astype(np.float32)
    out, pre = oracle.gemm_nt(A, sa, B, sb, want_pre=True)
    va = [[e4m3_exact(c) for c in row] for row in A]
    vb = [[e4m3_exact(c) for c in row] for row in B]
    fsa = [[Fraction(float(v)) for v in row] for row in sa]
    fsb = [[Fraction(float(v)) for v in row] for row in sb]
    for i in range(m):
        for j in range(n):
            terms = [va[i][t] * fsa[i][t // 128] * vb[j][t] * fsb[j // 128][t // 128]
                     for t in range(k)]
            tot = sum(terms)
            assert out[i, j] == bf16_nearest_exact(tot), (i, j)
            # FP64 evaluation: at most 2*KG roundings, each within 2^-53 of
            # the magnitude of the per-group terms
            per_group = [abs(sum(terms[128 * g:128 * g + 128])) for g in range(kg)]
            bound = 2 * kg * Fraction(1, 2 ** 53) * sum(per_group)
            assert abs(Fraction(pre[i, j]) - tot) <= bound, (i, j)


def test_p7_bruteforce_float64_medium():
    rng = np.random.default_rng(9)
    m, n, k = 64, 256, 256
    A = rand_finite_codes(rng, (m, k))
    B = rand_finite_codes(rng, (n, k))
    sa = rng.uniform(-1, 1, (m, 2)).astype(np.float32)
    sb = rng.uniform(-1, 1, (2, 2)).astype(np.float32)
    _, pre = oracle.gemm_nt(A, sa, B, sb, want_pre=True)
    deq_a = torch_e4m3_values(A) * np.repeat(sa.astype(np.float64), 128, axis=1)
    deq_b = torch_e4m3_values(B) * np.repeat(np.repeat(sb.astype(np.float64), 128, axis=0), 128, axis=1)
    direct = np.einsum("ik,jk->ij", deq_a.astype(np.longdouble), deq_b.astype(np.longdouble))
    np.testing.assert_allclose(pre, direct.astype(np.float64), rtol=1e-13, atol=1e-12 * np.abs(pre).max())


# ---- P8: unit scales against numpy's matmul --------------------------------------
def test_p8_unit_scales_equal_numpy_matmul():
    rng = np.random.default_rng(10)
    m, n, k = 33, 300, 640
    A = rand_finite_codes(rng, (m, k))
    B = rand_finite_codes(rng, (n, k))
    out = oracle.gemm_nt(A, np.ones((m, 5), np.float32), B, np.ones((3, 5), np.float32))
    d = torch_e4m3_values(A) @ torch_e4m3_values(B).T      # exact: multiples of 2^-18 < 2^53
    ref = torch.tensor(d).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, oracle.bf16_rne(d))
    same = np.float32(d).astype(np.float64) == d
    assert np.array_equal(out[same], ref[same])
    # codes of small integers: every sum is exact in fp32, so torch's own
    # fp32 -> bf16 rounding pins every element
    codes = torch_e4m3_encode(np.arange(-8, 9, dtype=np.float32))
    A2 = codes[rng.integers(0, 17, (m, k))]
    B2 = codes[rng.integers(0, 17, (n, k))]
    out2 = oracle.gemm_nt(A2, np.ones((m, 5), np.float32), B2, np.ones((3, 5), np.float32))
    d2 = torch_e4m3_values(A2) @ torch_e4m3_values(B2).T
    assert np.all(np.float32(d2).astype(np.float64) == d2)
    ref2 = torch.tensor(d2).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out2, ref2)


# ---- P9: sanity band against the unquantised product ------------------------------
def test_p9_quantised_vs_fp32_band():
    m, n, k = 64, 256, 1024
    x, w = synth.dense_operands(m, n, k, seed=0)
    qa, sa = oracle.cast_1x128(x)
    qb, sb = oracle.cast_128x128(w)
    out = oracle.bf16_bits_to_f64(oracle.gemm_nt(qa, sa, qb, sb))
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert 1e-3 < rel < 1e-1, rel


# ---- P10: cast invariants and the pages' cast via torch ----------------------------
def _torch_cast_1x128(x):
    """The kwkr.cn §4.2 snippet per 1x128 group: scale = amax / 448,
    q = (x / scale).to(float8_e4m3fn) (fp32 torch ops on the CPU)."""
    m, k = x.shape
    kg = (k + 127) // 128
    q = np.empty((m, k), np.uint8)
    s = np.empty((m, kg), np.float32)
    xt = torch.tensor(x)
    for g in range(kg):
        blk = xt[:, 128 * g:128 * g + 128]
        amax = blk.abs().amax(dim=1, keepdim=True)
        sc = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
        q[:, 128 * g:128 * g + 128] = (blk / sc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        s[:, g] = sc[:, 0].numpy()
    return q, s


def test_p10_cast_matches_torch_and_invariants():
    x = synth.normal_f32(0, 1, (37, 1000))        # partial last group
    x[5, :] = 0.0                                  # all-zero row
    x[6, 128:256] = 0.0                            # one zero group
    x[7, 3] = -0.0
    q, s = oracle.cast_1x128(x)
    tq, ts = _torch_cast_1x128(x)
    assert np.array_equal(s, ts)
    assert np.array_equal(q, tq)
    assert np.all(s[5] == 1.0) and np.all(q[5] == 0) and s[6, 1] == 1.0
    t = oracle.e4m3_table()
    for i in range(x.shape[0]):
        for g in range(s.shape[1]):
            blk = x[i, 128 * g:128 * g + 128]
            qb = q[i, 128 * g:128 * g + 128]
            if np.abs(blk).max() > 0:
                am = np.abs(blk) == np.abs(blk).max()
                assert np.all((qb[am] & 0x7F) == 0x7E)
            y = blk.astype(np.float64) / s[i, g]
            dq = t[qb]
            # half an E4M3 ulp at y (the spacing of the binade holding |y|)
            e = np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6)))
            half_ulp = 2.0 ** (e - 3) / 2
            assert np.all(np.abs(dq - y) <= half_ulp * (1 + 1e-6) + 1e-30)


def test_p10_bf16_input_cast_equals_f32_cast():
    x = synth.normal_f32(0, 1, (9, 384))
    xb = torch.tensor(x).to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    q1, s1 = oracle.cast_1x128(bits)
    q2, s2 = oracle.cast_1x128(xb.to(torch.float32).numpy())
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_p10_block_cast_edges():
    w = synth.normal_f32(0, 2, (130, 200))
    w[128:, 128:] *= 100.0                 # the 2x72 corner block
    q, s = oracle.cast_128x128(w)
    assert s.shape == (2, 2)
    assert s[1, 1] == np.float32(np.abs(w[128:, 128:]).max() / np.float32(448.0))
    assert s[0, 1] == np.float32(np.abs(w[:128, 128:]).max() / np.float32(448.0))
    for b, g in [(0, 0), (0, 1), (1, 0), (1, 1)]:
        blk = w[128 * b:128 * b + 128, 128 * g:128 * g + 128]
        tq = (torch.tensor(blk) / torch.tensor(s[b, g])).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(q[128 * b:128 * b + 128, 128 * g:128 * g + 128], tq)


# ---- P11: grouped layouts reduce to the dense definition ---------------------------
def test_p11_contiguous_equals_dense_per_expert():
    sizes = [128, 256, 128]
    n, k = 136, 256
    x, w, m_idx = synth.contiguous_operands(sizes, n, k, seed=3)
    qa, sa = oracle.cast_1x128(x)
    qb = np.empty(w.shape, np.uint8)
    sb = np.empty((3, 2, 2), np.float32)
    for g in range(3):
        qb[g], sb[g] = oracle.cast_128x128(w[g])
    m_idx = m_idx.copy()
    m_idx[128:256] = -1                                   # a skipped block
    out = np.full((512, n), 0xABCD, np.uint16)
    oracle.gemm_contiguous(qa, sa, qb, sb, m_idx, out)
    assert np.all(out[128:256] == 0xABCD)
    r0 = 0
    for g, sz in enumerate(sizes):
        rows = slice(r0, r0 + sz)
        want = oracle.gemm_nt(qa[rows], sa[rows], qb[g], sb[g])
        if g == 1:
            want[:128] = 0xABCD
        assert np.array_equal(out[rows], want)
        r0 += sz


def test_p11_masked_equals_dense_on_valid_rows():
    G, max_m, n, k = 3, 40, 64, 256
    x, w = synth.masked_operands(G, max_m, n, k, seed=4)
    counts = np.array([0, 17, 40], np.int32)
    qa = np.empty((G, max_m, k), np.uint8)
    sa = np.empty((G, max_m, 2), np.float32)
    qb = np.empty((G, n, k), np.uint8)
    sb = np.empty((G, 1, 2), np.float32)
    for g in range(G):
        qa[g], sa[g] = oracle.cast_1x128(x[g])
        qb[g], sb[g] = oracle.cast_128x128(w[g])
    ga = synth.garbage_bytes(qa.size, seed=4).reshape(qa.shape)
    gs = synth.garbage_bytes(sa.size * 4, seed=5).view(np.float32).reshape(sa.shape)
    for g in range(G):
        c = counts[g]
        qa[g, c:] = ga[g, c:]          # may hold NaN codes
        sa[g, c:] = gs[g, c:]          # may hold NaN/Inf bit patterns
    out = np.full((G, max_m, n), 0x5A5A, np.uint16)
    oracle.gemm_masked(qa, sa, qb, sb, np.array([0, 17, 99], np.int32), out)  # 99 clamps to 40
    assert np.all(out[0] == 0x5A5A) and np.all(out[1, 17:] == 0x5A5A)
    for g in (1, 2):
        c = counts[g]
        assert np.array_equal(out[g, :c], oracle.gemm_nt(qa[g, :c], sa[g, :c], qb[g], sb[g]))


def test_points_equal_full_gemm():
    rng = np.random.default_rng(11)
    m, n, k = 20, 300, 384
    A = rand_finite_codes(rng, (m, k))
    B = rand_finite_codes(rng, (n, k))
    sa = rng.standard_normal((m, 3)).astype(np.float32)
    sb = rng.standard_normal((3, 3)).astype(np.float32)
    full = oracle.gemm_nt(A, sa, B, sb)
    rows = rng.integers(0, m, 500)
    cols = rng.integers(0, n, 500)
    assert np.array_equal(oracle.gemm_points(A, sa, B, sb, rows, cols), full[rows, cols])


def test_tolerance_check_catches_a_planted_error():
    """A mistake planted in an oracle-side result: one element off by 5% of
    rms must fail the bar, one off by 0.1% of rms must pass."""
    rng = np.random.default_rng(12)
    ref = rng.standard_normal(4096)
    ref_bits = oracle.bf16_rne(ref)
    ok, _, rms = oracle.tolerance_check(ref_bits, ref_bits)
    assert ok
    bad = ref.copy(); bad[17] += 0.05 * rms
    assert not oracle.tolerance_check(oracle.bf16_rne(bad), ref_bits)[0]
    fine = ref.copy(); fine[17] += 0.001 * rms
    assert oracle.tolerance_check(oracle.bf16_rne(fine), ref_bits)[0]
    nan = ref.copy(); nan[3] = np.nan
    assert not oracle.tolerance_check(oracle.bf16_rne(nan), ref_bits)[0]


# ---- E5M2 (the second format: "DeepGEMM: FP8 GEMM kernel optimisation
# practice on Hopper Tensor Cores" §1.3 and the §3.1 table) ---------------------
def torch_e5m2_values(codes):
    t = torch.tensor(np.asarray(codes, np.uint8)).view(torch.float8_e5m2)
    return t.to(torch.float64).numpy()


def torch_e5m2_encode(x):
    """torch's float32 -> float8_e5m2 conversion (round to nearest even)."""
    t = torch.tensor(np.asarray(x, np.float32)).to(torch.float8_e5m2)
    return t.view(torch.uint8).numpy()


def test_e5m2_decode_closed_forms_and_torch():
    t = oracle.fp8_table(oracle.E5M2)
    assert t[0x7B] == 57344.0 and t[0x04] == 2.0 ** -14 and t[0x01] == 2.0 ** -16 and t[0x3C] == 1.0
    assert np.isposinf(t[0x7C]) and np.isneginf(t[0xFC])
    assert np.all(np.isnan(t[[0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]]))
    assert np.all(np.diff(t[:0x7C]) > 0)
    ref = torch_e5m2_values(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(t), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(t[fin], ref[fin])
    # the E4M3 table is unchanged by the format argument
    assert np.array_equal(oracle.fp8_table(oracle.E4M3), oracle.e4m3_table(), equal_nan=True)


def test_e5m2_encode_roundtrip_midpoints_saturation():
    t = oracle.fp8_table(oracle.E5M2)
    codes = np.array([c for c in range(256) if np.isfinite(t[c])], np.uint8)
    assert np.array_equal(oracle.fp8_encode(t[codes], oracle.E5M2), codes)
    for c in range(0, 0x7B):
        mid = (t[c] + t[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert oracle.fp8_encode([mid], oracle.E5M2)[0] == want, hex(c)
    q = oracle.fp8_encode([57344.0, 61439.0, 61440.0, 1e30, np.inf, -7e4, np.nan], oracle.E5M2)
    assert list(q) == [0x7B, 0x7B, 0x7B, 0x7B, 0x7B, 0xFB, 0x7F]


def test_e5m2_encode_matches_torch_and_bruteforce():
    rng = np.random.default_rng(2)
    t = oracle.fp8_table(oracle.E5M2)
    x = np.concatenate([
        rng.standard_normal(20000) * 3000,
        np.exp(rng.uniform(np.log(1e-7), np.log(57000.0), 20000)) * rng.choice([-1, 1], 20000),
    ]).astype(np.float32)
    mids = ((t[:0x7B] + t[1:0x7C]) / 2).astype(np.float32)
    near = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e5))])
    x = np.concatenate([x, near, -near, mids]).astype(np.float32)
    x = x[np.abs(x) <= 57344.0]  # torch's conversion is not saturating past the maximum
    ours = oracle.fp8_encode(x.astype(np.float64), oracle.E5M2)
    assert np.array_equal(ours, torch_e5m2_encode(x))
    fin = [(Fraction(float(t[c])), c) for c in range(0x7C)]
    for idx in range(0, x.size, 97):
        v = x[idx]
        a = Fraction(float(abs(v)))
        best = min(fin, key=lambda p: (abs(p[0] - a), p[1] % 2))
        assert ours[idx] == best[1] | (0x80 if np.signbit(v) else 0)


def test_e5m2_cast_matches_torch_reference():
    """The cast with the E5M2 maximum, against the usage-article cast code
    (amax / max, x / scale, convert) run with torch on the CPU."""
    x = synth.normal_f32(3, 1, (29, 700))
    x[4, :] = 0.0
    q, s = oracle.cast_1x128(x, fmt=oracle.E5M2)
    xt = torch.tensor(x)
    kg = s.shape[1]
    for g in range(kg):
        blk = xt[:, 128 * g:128 * g + 128]
        amax = blk.abs().amax(dim=1)
        sc = torch.where(amax == 0, torch.ones_like(amax), amax / 57344.0)
        assert np.array_equal(s[:, g], sc.numpy())
        y = (blk / sc[:, None]).to(torch.float8_e5m2).view(torch.uint8).numpy()
        assert np.array_equal(q[:, 128 * g:128 * g + 128], y)
    wq, ws = oracle.cast_128x128(synth.normal_f32(4, 2, (200, 260)), fmt=oracle.E5M2)
    assert ws.shape == (2, 3) and np.all((wq & 0x7F) <= 0x7B)


@pytest.mark.parametrize("a_fmt,b_fmt", [(1, 1), (0, 1), (1, 0)])
def test_e5m2_gemm_bruteforce_rational(a_fmt, b_fmt):
    """Mixed and pure E5M2 operands: exact rational sums (partial K group
    and N block), decoded through torch's own format tables."""
    rng = np.random.default_rng(10 + a_fmt * 2 + b_fmt)
    m, n, k = 3, 130, 259
    kg, nb = 3, 2

    def codes(fmt, shape):
        c = rng.integers(0, 256, size=shape, dtype=np.uint8)
        if fmt == 1:
            c[(c & 0x7C) == 0x7C] &= 0xF3        # no inf / NaN codes
        else:
            c[(c & 0x7F) == 0x7F] &= 0xFE
        return c

    A, B = codes(a_fmt, (m, k)), codes(b_fmt, (n, k))
    sa = rng.standard_normal((m, kg)).astype(np.float32)
    sb = rng.standard_normal((nb, kg)).astype(np.float32)
    out = oracle.gemm_nt(A, sa, B, sb, a_fmt=a_fmt, b_fmt=b_fmt)
    dec = {0: torch_e4m3_values, 1: torch_e5m2_values}
    va = [[Fraction(float(v)) for v in dec[a_fmt](row)] for row in A]
    vb = [[Fraction(float(v)) for v in dec[b_fmt](row)] for row in B]
    for i in range(m):
        for j in range(0, n, 3):
            tot = sum(va[i][t] * Fraction(float(sa[i, t // 128])) * vb[j][t] * Fraction(float(sb[j // 128, t // 128]))
                      for t in range(k))
            assert out[i, j] == bf16_nearest_exact(tot), (i, j)


def test_group_sum_is_exact_where_fp64_summation_is_not():
    """E5M2 products span 2^-32 .. 2^31.6, so a group sum can need ~71
    significant bits: summed left to right in FP64, 2^30 + 2^-32 - 2^30
    loses the small term.  The oracle sums each K group exactly and rounds
    once, so it returns 2^-32 (as exact rational arithmetic does)."""
    k = 128
    A = np.zeros((1, k), np.uint8)
    B = np.zeros((1, k), np.uint8)
    big, tiny, neg_big = 0x78, 0x01, 0xF8            # E5M2: 2^15, 2^-16, -2^15
    A[0, :3] = [big, tiny, neg_big]
    B[0, :3] = [big, tiny, big]
    one = np.ones((1, 1), np.float32)
    dec = oracle.fp8_table(oracle.E5M2)
    assert dec[big] == 2.0 ** 15 and dec[tiny] == 2.0 ** -16 and dec[neg_big] == -2.0 ** 15
    out, pre = oracle.gemm_nt(A, one, B, one, want_pre=True, a_fmt=oracle.E5M2, b_fmt=oracle.E5M2)
    assert pre[0, 0] == 2.0 ** -32
    assert out[0, 0] == oracle.bf16_rne(2.0 ** -32)
    # the same cancellation spread over a mixed-format pair (E4M3 x E5M2):
    # 448 * 2^15, then 2^-9 * 2^-16, then -448 * 2^15
    A4 = np.zeros((1, k), np.uint8)
    A4[0, :3] = [0x7E, 0x01, 0xFE]                    # E4M3: 448, 2^-9, -448
    out, pre = oracle.gemm_nt(A4, one, B, one, want_pre=True, a_fmt=oracle.E4M3, b_fmt=oracle.E5M2)
    assert pre[0, 0] == 2.0 ** -25


def test_group_sum_propagates_nonfinite_codes():
    """A NaN code (E4M3 0x7F) or an infinity (E5M2 0x7C) in a group makes
    that output NaN or infinite, as IEEE arithmetic on the decoded values."""
    k = 256
    A = np.full((2, k), 0x38, np.uint8)               # 1.0
    B = np.full((1, k), 0x38, np.uint8)
    A[0, 5] = 0x7F
    one = np.ones((2, 2), np.float32)
    _, pre = oracle.gemm_nt(A, one, B, one[:1], want_pre=True)
    assert np.isnan(pre[0, 0]) and pre[1, 0] == 256.0
    A5 = np.full((1, k), 0x3C, np.uint8)              # E5M2 1.0
    A5[0, 200] = 0x7C                                 # +inf
    _, pre = oracle.gemm_nt(A5, one[:1], B, one[:1], want_pre=True, a_fmt=oracle.E5M2, b_fmt=oracle.E4M3)
    assert pre[0, 0] == np.inf
