"""CPU oracle for the block-scaled FP8 GEMM path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The GPU library never does,
and this package never imports the GPU library.  The arithmetic lives in
``fp8_oracle.cpp`` (plain loops, FP64 accumulation, one BF16 rounding); this
module only builds that file with g++ and marshals numpy arrays into it.

Parity unpinned: nothing here is unpinned.  Every exported function is pinned
by ``tests/test_oracle_pins.py`` against closed forms, exact integer or
rational recomputation, brute force or a numpy library routine.

Logical scale layouts: LHS scales ``[rows][KG]``, RHS scales ``[NB][KG]``,
with ``KG = ceil(k/128)`` and ``NB = ceil(n/128)``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8_oracle.cpp")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int


def build() -> str:
    """Compile the oracle with g++ (no fast-math, no FP contraction)."""
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread",
           "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", _SO + ".tmp"]
    subprocess.check_call(cmd)
    os.replace(_SO + ".tmp", _SO)
    return _SO


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_SO)
    lib.orc_e4m3_table.argtypes = [_f64p]
    lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_e4m3_encode_array.argtypes = [_f64p, _i64, _u8p]
    lib.orc_bf16_rne.argtypes = [ctypes.c_double]
    lib.orc_bf16_rne.restype = ctypes.c_uint16
    lib.orc_bf16_rne_array.argtypes = [_f64p, _i64, _u16p]
    lib.orc_fp8_table.argtypes = [_int, _f64p]
    lib.orc_fp8_encode_array.argtypes = [_int, _f64p, _i64, _u8p]
    lib.orc_cast_1x128_f32.argtypes = [_f32p, _i64, _i64, _u8p, _f32p, _int, _int]
    lib.orc_cast_1x128_bf16.argtypes = [_u16p, _i64, _i64, _u8p, _f32p, _int, _int]
    lib.orc_cast_128x128_f32.argtypes = [_f32p, _i64, _i64, _u8p, _f32p, _int, _int]
    lib.orc_gemm_nt.argtypes = [_u8p, _f32p, _u8p, _f32p, _i64, _i64, _i64,
                                _u16p, _vp, _int, _int, _int]
    lib.orc_gemm_contiguous.argtypes = [_u8p, _f32p, _u8p, _f32p, _i32p, _i64,
                                        _i64, _i64, _i64, _u16p, _vp, _int]
    lib.orc_gemm_masked.argtypes = [_u8p, _f32p, _u8p, _f32p, _i32p, _i64,
                                    _i64, _i64, _i64, _u16p, _vp, _int]
    lib.orc_gemm_points.argtypes = [_u8p, _f32p, _u8p, _f32p, _i64, _i64p,
                                    _i64p, _i64, _u16p, _vp, _int, _int, _int]
    lib.orc_hardware_threads.restype = _int
    _lib = lib
    return lib


def hardware_threads() -> int:
    return int(_load().orc_hardware_threads())


def _threads(nthreads):
    return int(nthreads) if nthreads else hardware_threads()


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _pre_ptr(pre):
    return None if pre is None else pre.ctypes.data_as(ctypes.c_void_p)


def kg_of(k: int) -> int:
    return (int(k) + 127) // 128


E4M3, E5M2 = 0, 1  # FP8 formats


def fp8_table(fmt=E4M3) -> np.ndarray:
    """Value of each of the 256 codes of the format (E4M3FN: NaN for 0x7F and
    0xFF; E5M2: +-inf for 0x7C / 0xFC, NaN for 0x7D-0x7F and 0xFD-0xFF)."""
    out = np.empty(256, np.float64)
    _load().orc_fp8_table(int(fmt), out)
    return out


def fp8_encode(x, fmt=E4M3) -> np.ndarray:
    """Round to the nearest code of the format, ties to even, saturating at
    its largest finite value (448 or 57344)."""
    xa = _c(np.asarray(x, np.float64).ravel(), np.float64)
    q = np.empty(xa.size, np.uint8)
    _load().orc_fp8_encode_array(int(fmt), xa, xa.size, q)
    return q.reshape(np.shape(x))


# --------------------------------------------------------------------------
def e4m3_table() -> np.ndarray:
    """Value of each of the 256 E4M3FN codes (NaN for 0x7F and 0xFF)."""
    out = np.empty(256, np.float64)
    _load().orc_e4m3_table(out)
    return out


def e4m3_encode(x) -> np.ndarray:
    """Round to nearest E4M3FN code, ties to even, saturating at +-448."""
    xa = _c(np.asarray(x, np.float64).ravel(), np.float64)
    q = np.empty(xa.size, np.uint8)
    _load().orc_e4m3_encode_array(xa, xa.size, q)
    return q.reshape(np.shape(x))


def bf16_rne(x) -> np.ndarray:
    """BF16 bit patterns of x (FP64 in), rounded once to nearest-even."""
    xa = _c(np.asarray(x, np.float64).ravel(), np.float64)
    out = np.empty(xa.size, np.uint16)
    _load().orc_bf16_rne_array(xa, xa.size, out)
    return out.reshape(np.shape(x))


def cast_1x128(x, nthreads=None, fmt=E4M3):
    """Per-token-group cast: x [m][k] fp32 (or uint16 bf16 bits) ->
    (codes uint8 [m][k], scales fp32 [m][KG])."""
    x = np.asarray(x)
    m, k = x.shape
    q = np.empty((m, k), np.uint8)
    s = np.empty((m, kg_of(k)), np.float32)
    if x.dtype == np.uint16:
        _load().orc_cast_1x128_bf16(_c(x, np.uint16), m, k, q, s, _threads(nthreads), int(fmt))
    else:
        _load().orc_cast_1x128_f32(_c(x, np.float32), m, k, q, s, _threads(nthreads), int(fmt))
    return q, s


def cast_128x128(w, nthreads=None, fmt=E4M3):
    """128x128 block cast: w [n][k] fp32 -> (codes [n][k], scales [NB][KG])."""
    w = _c(w, np.float32)
    n, k = w.shape
    q = np.empty((n, k), np.uint8)
    s = np.empty(((n + 127) // 128, kg_of(k)), np.float32)
    _load().orc_cast_128x128_f32(w, n, k, q, s, _threads(nthreads), int(fmt))
    return q, s


def gemm_nt(A, sa, B, sb, want_pre=False, nthreads=None, a_fmt=E4M3, b_fmt=E4M3):
    """Dense NT GEMM -> bf16 bits [m][n] (and the FP64 pre-rounding values).
    a_fmt / b_fmt: the operands' FP8 formats."""
    A = _c(A, np.uint8); B = _c(B, np.uint8)
    m, k = A.shape
    n = B.shape[0]
    out = np.empty((m, n), np.uint16)
    pre = np.empty((m, n), np.float64) if want_pre else None
    _load().orc_gemm_nt(A, _c(sa, np.float32), B, _c(sb, np.float32), m, n, k,
                        out, _pre_ptr(pre), _threads(nthreads), int(a_fmt), int(b_fmt))
    return (out, pre) if want_pre else out


def gemm_contiguous(A, sa, B, sb, m_indices, out, want_pre=False, nthreads=None):
    """Contiguous grouped GEMM into ``out`` ([M][n] uint16, rows with a
    negative group index untouched).  B [G][n][k], sb [G][NB][KG]."""
    A = _c(A, np.uint8); B = _c(B, np.uint8)
    M, k = A.shape
    G, n, _ = B.shape
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.shape == (M, n)
    pre = np.full((M, n), np.nan) if want_pre else None
    _load().orc_gemm_contiguous(A, _c(sa, np.float32), B, _c(sb, np.float32),
                                _c(m_indices, np.int32), M, n, k, G, out,
                                _pre_ptr(pre), _threads(nthreads))
    return pre


def gemm_masked(A, sa, B, sb, masked_m, out, want_pre=False, nthreads=None):
    """Masked grouped GEMM into ``out`` ([G][max_m][n] uint16; rows at or past
    each group's count untouched).  A [G][max_m][k], sa [G][max_m][KG]."""
    A = _c(A, np.uint8); B = _c(B, np.uint8)
    G, max_m, k = A.shape
    n = B.shape[1]
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.shape == (G, max_m, n)
    pre = np.full((G, max_m, n), np.nan) if want_pre else None
    _load().orc_gemm_masked(A, _c(sa, np.float32), B, _c(sb, np.float32),
                            _c(masked_m, np.int32), G, max_m, n, k, out,
                            _pre_ptr(pre), _threads(nthreads))
    return pre


def gemm_points(A, sa, B, sb, rows, cols, want_pre=False, nthreads=None, a_fmt=E4M3, b_fmt=E4M3):
    """Selected outputs (rows[p], cols[p]) of A . B^T for one RHS."""
    A = _c(A, np.uint8); B = _c(B, np.uint8)
    k = A.shape[-1]
    rows = _c(rows, np.int64); cols = _c(cols, np.int64)
    assert rows.shape == cols.shape
    out = np.empty(rows.size, np.uint16)
    pre = np.empty(rows.size, np.float64) if want_pre else None
    _load().orc_gemm_points(A.reshape(-1, k), _c(sa, np.float32).reshape(A.reshape(-1, k).shape[0], -1),
                            B.reshape(-1, k), _c(sb, np.float32), k, rows, cols,
                            rows.size, out, _pre_ptr(pre), _threads(nthreads), int(a_fmt), int(b_fmt))
    return (out, pre) if want_pre else out


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns to float64 (exact)."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def tolerance_check(gpu_bits, ref_bits, rtol=8e-3, atol_rms=1e-2):
    """The parity bar: |gpu - ref| <= rtol*|ref| + atol_rms*rms(ref), taken
    elementwise over the given (valid) outputs; any NaN/Inf in either fails.
    Returns (ok, worst_ratio, rms)."""
    g = bf16_bits_to_f64(gpu_bits).ravel()
    r = bf16_bits_to_f64(ref_bits).ravel()
    if g.size == 0:
        return True, 0.0, 0.0
    if not (np.isfinite(g).all() and np.isfinite(r).all()):
        return False, float("inf"), float("nan")
    rms = float(np.sqrt(np.mean(r * r)))
    bound = rtol * np.abs(r) + atol_rms * rms
    ratio = np.abs(g - r) / np.where(bound > 0, bound, 1.0)
    worst = float(ratio.max())
    return bool(worst <= 1.0), worst, rms


# MoE layout steps (plain numpy, see moe.py)
from .moe import (moe_contiguous_rows, moe_counts, moe_gather_rows, moe_layout_contiguous,  # noqa: E402,F401
                  moe_layout_masked, moe_ranks, moe_scatter_rows)
