"""Seeded synthetic inputs shared by the tests and the benchmark.

This module draws random numbers and arranges them into the workloads'
shapes; it holds none of the GEMM or cast arithmetic.  Everything is
counter-based, so any slice of any stream can be regenerated independently:

* splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): output i of a stream is
  ``mix64(key + (i + 1) * 0x9E3779B97F4A7C15)``.
* A stream is named by ``(seed, stream_id)``; its key is
  ``mix64(seed * 0x9E3779B97F4A7C15 + stream_id)``.
* Uniform doubles in (0, 1] are ``((u >> 11) + 1) * 2^-53``.
* Normal draws use the Box-Muller transform on consecutive uniform pairs
  (u1, u2): ``r = sqrt(-2 ln u1)``, ``z0 = r cos(2 pi u2)``,
  ``z1 = r sin(2 pi u2)``, computed in float64 and then rounded to float32.
* Integers in [lo, hi] are ``lo + (((u >> 11) * (hi - lo + 1)) >> 53)``.

Stream ids used by the workloads: 1 LHS values, 2 RHS values, 3 contiguous
group sizes, 4 masked counts, 5 garbage bytes for masked rows past the count,
6 LHS outlier mask, 7 RHS outlier mask.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22

S_LHS, S_RHS, S_GROUP_SIZES, S_MASKED_COUNTS, S_GARBAGE, S_OUT_LHS, S_OUT_RHS = 1, 2, 3, 4, 5, 6, 7


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _key(seed: int, stream: int) -> np.uint64:
    with np.errstate(over="ignore"):
        z = np.array([np.uint64(seed) * GAMMA + np.uint64(stream)], np.uint64)
        return _mix64(z)[0]


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _chunked(total: int, fn, out: np.ndarray):
    """Fill out[0:total] by fn(start, stop) over chunks, in parallel threads
    (numpy releases the GIL inside its array loops)."""
    starts = list(range(0, total, _CHUNK))
    if len(starts) <= 1:
        if total:
            out[:total] = fn(0, total)
        return out

    def run(s):
        e = min(s + _CHUNK, total)
        out[s:e] = fn(s, e)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(run, starts))
    return out


def raw_u64(seed: int, stream: int, count: int, offset: int = 0) -> np.ndarray:
    """Outputs offset .. offset+count-1 of the splitmix64 stream."""
    key = _key(seed, stream)

    def fn(s, e):
        with np.errstate(over="ignore"):
            ctr = np.arange(offset + s + 1, offset + e + 1, dtype=np.uint64)
            return _mix64(key + ctr * GAMMA)

    return _chunked(count, fn, np.empty(count, np.uint64))


def _uniform_from(u: np.ndarray) -> np.ndarray:
    return ((u >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)


def uniform(seed: int, stream: int, count: int) -> np.ndarray:
    """Uniform float64 in (0, 1]."""
    return _uniform_from(raw_u64(seed, stream, count))


def normal_f32(seed: int, stream: int, shape) -> np.ndarray:
    """N(0, 1) float32 array of the given shape (Box-Muller)."""
    count = int(np.prod(shape, dtype=np.int64))
    pairs = (count + 1) // 2
    key = _key(seed, stream)

    def fn(s, e):  # s, e index pairs
        with np.errstate(over="ignore"):
            ctr = np.arange(2 * s + 1, 2 * e + 1, dtype=np.uint64)
            u = _uniform_from(_mix64(key + ctr * GAMMA))
        u1, u2 = u[0::2], u[1::2]
        r = np.sqrt(-2.0 * np.log(u1))
        th = (2.0 * np.pi) * u2
        z = np.empty(2 * (e - s), np.float32)
        z[0::2] = r * np.cos(th)
        z[1::2] = r * np.sin(th)
        return z.reshape(e - s, 2)

    flat = _chunked(pairs, fn, np.empty((pairs, 2), np.float32)).reshape(-1)
    return flat[:count].reshape(shape)


def randint(seed: int, stream: int, count: int, lo: int, hi: int) -> np.ndarray:
    """Integers uniform in [lo, hi] (inclusive), int64."""
    span = np.uint64(hi - lo + 1)
    u = raw_u64(seed, stream, count) >> np.uint64(11)
    with np.errstate(over="ignore"):
        v = (u * span) >> np.uint64(53)
    return v.astype(np.int64) + lo


def random_bytes(seed: int, stream: int, count: int) -> np.ndarray:
    """count uniformly random bytes."""
    words = raw_u64(seed, stream, (count + 7) // 8)
    return words.view(np.uint8)[:count].copy()


def with_outliers(x: np.ndarray, seed: int, stream: int, p: float = 0.01,
                  factor: float = 50.0) -> np.ndarray:
    """Multiply each element by `factor` independently with probability p."""
    u = uniform(seed, stream, x.size).reshape(x.shape)
    return np.where(u <= p, x * np.float32(factor), x).astype(np.float32)


# ---- workload recipes ------------------------------------------------------
def dense_operands(m: int, n: int, k: int, seed: int = 0, outliers: bool = False):
    """fp32 activations x [m][k] and weights w [n][k], N(0, 1)."""
    x = normal_f32(seed, S_LHS, (m, k))
    w = normal_f32(seed, S_RHS, (n, k))
    if outliers:
        x = with_outliers(x, seed, S_OUT_LHS)
        w = with_outliers(w, seed, S_OUT_RHS)
    return x, w


def contiguous_group_sizes(groups: int = 8, seed: int = 0, lo: int = 4, hi: int = 32):
    """Rows per expert: 128 * U{lo..hi}."""
    return 128 * randint(seed, S_GROUP_SIZES, groups, lo, hi)


def contiguous_operands(sizes, n: int, k: int, seed: int = 0):
    """Rows of all experts concatenated along M in expert order.
    Returns x [M][k] fp32, w [G][n][k] fp32 and m_indices [M] int32."""
    sizes = np.asarray(sizes, np.int64)
    M = int(sizes.sum())
    G = sizes.size
    x = normal_f32(seed, S_LHS, (M, k))
    w = normal_f32(seed, S_RHS, (G, n, k))
    m_indices = np.repeat(np.arange(G, dtype=np.int32), sizes)
    return x, w, m_indices


def masked_counts(groups: int = 16, max_m: int = 256, seed: int = 0):
    """Valid rows per group, uniform in [0, max_m]."""
    return randint(seed, S_MASKED_COUNTS, groups, 0, max_m).astype(np.int32)


def masked_operands(groups: int, max_m: int, n: int, k: int, seed: int = 0):
    """x [G][max_m][k] fp32 (every row drawn; rows past the count are later
    overwritten with garbage bytes) and w [G][n][k] fp32."""
    x = normal_f32(seed, S_LHS, (groups, max_m, k))
    w = normal_f32(seed, S_RHS, (groups, n, k))
    return x, w


def garbage_bytes(count: int, seed: int = 0) -> np.ndarray:
    return random_bytes(seed, S_GARBAGE, count)
