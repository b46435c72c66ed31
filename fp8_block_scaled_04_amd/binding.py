"""ctypes binding of libfp8gemm.so, with the C ABI's names.

Argument marshalling only: tensors are PyTorch device tensors (PyTorch is
used for device memory and streams); every step of the computation runs in
the library's HIP kernels.  There is no fallback path: if the library is
missing, every call raises.

Layouts (see include/fp8gemm.h): FP8 tensors are uint8 (or
torch.float8_e4m3fn) codes; LHS scales are MN-major ``[KG][ld]`` float32;
RHS scales ``[NB][KG]`` (``[G][NB][KG]`` grouped) float32; outputs bfloat16.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

from . import build as _build

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = _build.LIB
HEADER = os.path.join(os.path.dirname(HERE), "include", "fp8gemm.h")

FP8G_OK, FP8G_EINVAL, FP8G_EUNSUPPORTED, FP8G_ELAUNCH, FP8G_ESCRATCH = 0, -1, -2, -3, -4
FP8G_F32, FP8G_BF16 = 0, 1
FP8G_E4M3, FP8G_E5M2 = 0, 1
FP8G_JIT_DENSE, FP8G_JIT_CONTIGUOUS, FP8G_JIT_MASKED = 0, 1, 2

_lib = None
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t


class Fp8GemmConfig(ctypes.Structure):
    """fp8_gemm_config: the tile configuration of a runtime-specialised GEMM."""
    _fields_ = [(f, ctypes.c_int) for f in ("block_m", "block_n", "waves_m", "waves_n", "waves_k", "stages",
                                          "k_per_stage", "splits", "specialize")]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}

    def __repr__(self):
        return f"Fp8GemmConfig({self.as_dict()})"


_cfgp = ctypes.POINTER(Fp8GemmConfig)

_SIGNATURES = {
    "fp8_gemm_nt": ([_vp, _vp, _i64, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp], _i32),
    "fp8_grouped_gemm_contiguous": ([_vp, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _sz, _vp], _i32),
    "fp8_grouped_gemm_masked": ([_vp, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _sz, _vp], _i32),
    "fp8_cast_per_token_group": ([_vp, _i32, _i32, _i32, _vp, _vp, _i64, _vp], _i32),
    "fp8_cast_per_block": ([_vp, _i32, _i32, _vp, _vp, _vp], _i32),
    "fp8_gemm_nt_noalloc": ([_vp, _vp, _i64, _vp, _vp, _vp, _i32, _i32, _i32, _vp], _i32),
    "fp8_gemm_describe": ([_i32, _i32, _i32, ctypes.c_char_p, _sz], _i32),
    "fp8_gemm_schedule": ([_i32, _i32, _i32, _i32, _i32, _vp, _vp, _i32], _i32),
    "fp8_gemm_nt_fmt": ([_vp, _i32, _vp, _i64, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp], _i32),
    "fp8_cast_per_token_group_fmt": ([_vp, _i32, _i32, _i32, _i32, _vp, _vp, _i64, _vp], _i32),
    "fp8_cast_per_block_fmt": ([_vp, _i32, _i32, _i32, _vp, _vp, _vp], _i32),
    "fp8_gemm_workspace_bytes": ([_i32, _i32, _i32, _i32], _sz),
    "fp8_set_num_cus": ([_i32], _i32),
    "fp8_get_num_cus": ([], _i32),
    "fp8_status_string": ([_i32], ctypes.c_char_p),
    "fp8_jit_default_config": ([_i32, _i32, _i32, _i32, _cfgp], _i32),
    "fp8_jit_config_supported": ([_i32, _cfgp], _i32),
    "fp8_jit_warmup": ([_i32, _i32, _i32, _i32, _i32, _cfgp], _i32),
    "fp8_jit_gemm_workspace_bytes": ([_i32, _i32, _i32, _cfgp], _sz),
    "fp8_jit_gemm_nt": ([_vp, _i32, _vp, _i64, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _cfgp, _vp, _sz, _vp], _i32),
    "fp8_jit_grouped_gemm_contiguous": ([_vp, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _cfgp, _vp],
                                        _i32),
    "fp8_jit_grouped_gemm_masked": ([_vp, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _cfgp, _vp], _i32),
    "fp8_jit_set_cache_dir": ([ctypes.c_char_p], _i32),
    "fp8_jit_get_cache_dir": ([ctypes.c_char_p, _sz], _i32),
    "fp8_jit_stats": ([ctypes.POINTER(ctypes.c_longlong), _i32], _i32),
    "fp8_moe_contiguous_rows": ([_i32, _i32], _i32),
    "fp8_moe_layout_workspace_bytes": ([_i32, _i32], _sz),
    "fp8_moe_layout_contiguous": ([_vp, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _sz, _vp], _i32),
    "fp8_moe_layout_masked": ([_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "fp8_moe_scatter_rows": ([_vp, _vp, _i64, _i32, _i32, _vp, _i32, _i32, _vp, _vp, _i64, _vp], _i32),
    "fp8_moe_gather_rows": ([_vp, _i32, _i32, _vp, _i32, _vp, _vp], _i32),
}


class Fp8GemmError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


def lib():
    """Load libfp8gemm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with fp8_block_scaled_04_amd.build.build()")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def header_functions():
    """Names of the functions declared in include/fp8gemm.h."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8_\w+)\s*\(", text)))


def status_string(status: int) -> str:
    return lib().fp8_status_string(int(status)).decode()


def _check(fn, status):
    if status != FP8G_OK:
        raise Fp8GemmError(fn, status)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


_FMT_DTYPES = {FP8G_E4M3: torch.float8_e4m3fn, FP8G_E5M2: torch.float8_e5m2}
_FMT_NAMES = {FP8G_E4M3: "E4M3", FP8G_E5M2: "E5M2"}


def _fmt(fmt, name):
    if fmt not in _FMT_DTYPES:
        raise ValueError(f"{name} must be FP8G_E4M3 or FP8G_E5M2, got {fmt!r}")
    return fmt


def _codes(t, name, fmt=FP8G_E4M3):
    if t.dtype == _FMT_DTYPES[fmt]:
        t = t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must hold {_FMT_NAMES[fmt]} codes (uint8 or {_FMT_DTYPES[fmt]}), got {t.dtype}")
    return _dev(t, name)


def _dev(t, name):
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _f32(t, name):
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    return _dev(t, name)


def _bf16(t, name):
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    return _dev(t, name)


def _i32t(t, name):
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32, got {t.dtype}")
    return _dev(t, name)


# ---- extent checks ---------------------------------------------------------
# The C ABI sees raw pointers only, so a tensor smaller than the sizes the
# call derives from lhs / rhs would be read or written out of bounds on the
# device.  Every tensor's shape and device is checked here, before the call.
def _kg(k):
    return (int(k) + 127) // 128


def _want(t, name, shape):
    if tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(v) for v in shape)}")


def _want_dim(t, name, dim):
    if t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dimensions, got shape {tuple(t.shape)}")


def _want_scales_mn(t, name, lead, rows):
    """MN-major LHS scales: shape lead + (ld,) with ld >= rows."""
    lead = tuple(int(v) for v in lead)
    if t.dim() != len(lead) + 1 or tuple(t.shape[:-1]) != lead or t.shape[-1] < rows:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {lead + ('ld',)} with ld >= {rows}")


def _same_device(**tensors):
    devs = {n: t.device for n, t in tensors.items() if t is not None}
    first = next(iter(devs.values()))
    for n, d in devs.items():
        if d != first:
            raise ValueError(f"{n} is on {d}, the other tensors on {first}")


def _workspace_ok(ws, name="workspace"):
    if ws is not None:
        _dev(ws, name)
    return ws


def _check_gemm_nt(lhs, lhs_scales, rhs, rhs_scales, out, workspace):
    _want_dim(lhs, "lhs", 2)
    _want_dim(rhs, "rhs", 2)
    m, k = lhs.shape
    n = rhs.shape[0]
    _want(rhs, "rhs", (n, k))
    _want_scales_mn(lhs_scales, "lhs_scales", (_kg(k),), m)
    _want(rhs_scales, "rhs_scales", (_kg(n), _kg(k)))
    _want(out, "out", (m, n))
    _workspace_ok(workspace)
    _same_device(lhs=lhs, lhs_scales=lhs_scales, rhs=rhs, rhs_scales=rhs_scales, out=out, workspace=workspace)
    return m, n, k


def _check_contiguous(lhs, lhs_scales, rhs, rhs_scales, out, m_indices):
    _want_dim(lhs, "lhs", 2)
    _want_dim(rhs, "rhs", 3)
    M, k = lhs.shape
    G, n = rhs.shape[0], rhs.shape[1]
    _want(rhs, "rhs", (G, n, k))
    _want_scales_mn(lhs_scales, "lhs_scales", (_kg(k),), M)
    _want(rhs_scales, "rhs_scales", (G, _kg(n), _kg(k)))
    _want(out, "out", (M, n))
    _want(m_indices, "m_indices", (M,))
    _same_device(lhs=lhs, lhs_scales=lhs_scales, rhs=rhs, rhs_scales=rhs_scales, out=out, m_indices=m_indices)
    return M, n, k, G


def _check_masked(lhs, lhs_scales, rhs, rhs_scales, out, masked_m):
    _want_dim(lhs, "lhs", 3)
    _want_dim(rhs, "rhs", 3)
    G, max_m, k = lhs.shape
    n = rhs.shape[1]
    _want(rhs, "rhs", (G, n, k))
    _want_scales_mn(lhs_scales, "lhs_scales", (G, _kg(k)), max_m)
    _want(rhs_scales, "rhs_scales", (G, _kg(n), _kg(k)))
    _want(out, "out", (G, max_m, n))
    _want(masked_m, "masked_m", (G,))
    _same_device(lhs=lhs, lhs_scales=lhs_scales, rhs=rhs, rhs_scales=rhs_scales, out=out, masked_m=masked_m)
    return G, max_m, n, k


def _check_cast(x, q, scales):
    _want_dim(x, "x", 2)
    m, k = x.shape
    _want(q, "q", (m, k))
    _want_scales_mn(scales, "scales", (_kg(k),), m)
    _same_device(x=x, q=q, scales=scales)
    return m, k


def _check_block_cast(w, q, scales):
    _want_dim(w, "w", 2)
    n, k = w.shape
    _want(q, "q", (n, k))
    _want(scales, "scales", (_kg(n), _kg(k)))
    _same_device(w=w, q=q, scales=scales)
    return n, k


# ---- entry points ------------------------------------------------------------
def fp8_gemm_nt(lhs, lhs_scales, rhs, rhs_scales, out, workspace=None, stream=None):
    """out[m][n] = block-scaled FP8 NT GEMM of lhs [m][k] and rhs [n][k].
    lhs_scales is MN-major [KG][ld >= m]; rhs_scales [NB][KG]."""
    lhs, rhs = _codes(lhs, "lhs"), _codes(rhs, "rhs")
    lhs_scales, rhs_scales = _f32(lhs_scales, "lhs_scales"), _f32(rhs_scales, "rhs_scales")
    out = _bf16(out, "out")
    m, n, k = _check_gemm_nt(lhs, lhs_scales, rhs, rhs_scales, out, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().fp8_gemm_nt(_p(lhs), _p(lhs_scales), lhs_scales.shape[-1], _p(rhs), _p(rhs_scales), _p(out),
                           m, n, k, _p(workspace), ws_bytes, _stream(stream))
    _check("fp8_gemm_nt", st)
    return out


def fp8_gemm_nt_noalloc(lhs, lhs_scales, rhs, rhs_scales, out, stream=None):
    """fp8_gemm_nt with no workspace and no allocation: split-K scratch is
    the library's static per-device array (calls on one device must not
    overlap)."""
    lhs, rhs = _codes(lhs, "lhs"), _codes(rhs, "rhs")
    lhs_scales, rhs_scales = _f32(lhs_scales, "lhs_scales"), _f32(rhs_scales, "rhs_scales")
    out = _bf16(out, "out")
    m, n, k = _check_gemm_nt(lhs, lhs_scales, rhs, rhs_scales, out, None)
    st = lib().fp8_gemm_nt_noalloc(_p(lhs), _p(lhs_scales), lhs_scales.shape[-1], _p(rhs), _p(rhs_scales), _p(out),
                                   m, n, k, _stream(stream))
    _check("fp8_gemm_nt_noalloc", st)
    return out


def fp8_gemm_nt_fmt(lhs, lhs_format, lhs_scales, rhs, rhs_format, rhs_scales, out, workspace=None, stream=None):
    """fp8_gemm_nt with each operand's format given (FP8G_E4M3 or FP8G_E5M2)."""
    lhs_format, rhs_format = _fmt(lhs_format, "lhs_format"), _fmt(rhs_format, "rhs_format")
    lhs, rhs = _codes(lhs, "lhs", lhs_format), _codes(rhs, "rhs", rhs_format)
    lhs_scales, rhs_scales = _f32(lhs_scales, "lhs_scales"), _f32(rhs_scales, "rhs_scales")
    out = _bf16(out, "out")
    m, n, k = _check_gemm_nt(lhs, lhs_scales, rhs, rhs_scales, out, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().fp8_gemm_nt_fmt(_p(lhs), lhs_format, _p(lhs_scales), lhs_scales.shape[-1], _p(rhs), rhs_format,
                               _p(rhs_scales), _p(out), m, n, k, _p(workspace), ws_bytes, _stream(stream))
    _check("fp8_gemm_nt_fmt", st)
    return out


# ---- runtime shape specialisation ---------------------------------------------
def _config(config, **overrides):
    """An Fp8GemmConfig from None (keep None), a config, or a dict of fields;
    keyword overrides replace fields."""
    if config is None and not overrides:
        return None
    c = Fp8GemmConfig()
    if isinstance(config, Fp8GemmConfig):
        ctypes.pointer(c)[0] = config
    elif isinstance(config, dict):
        for f, v in config.items():
            setattr(c, f, int(v))
    elif config is not None:
        raise TypeError("config must be an Fp8GemmConfig, a dict or None")
    for f, v in overrides.items():
        setattr(c, f, int(v))
    return c


def _cref(c):
    return None if c is None else ctypes.byref(c)


def fp8_jit_default_config(mode, m, n, k) -> Fp8GemmConfig:
    """The configuration the ahead-of-time path uses for this shape."""
    c = Fp8GemmConfig()
    _check("fp8_jit_default_config", lib().fp8_jit_default_config(mode, m, n, k, ctypes.byref(c)))
    return c


def fp8_jit_config_supported(mode, config) -> bool:
    return lib().fp8_jit_config_supported(mode, _cref(_config(config))) == FP8G_OK


def fp8_jit_warmup(mode, n, k, lhs_format=FP8G_E4M3, rhs_format=FP8G_E4M3, config=None):
    """Compile (or read from the cache) and load a kernel without launching it."""
    _check("fp8_jit_warmup", lib().fp8_jit_warmup(mode, n, k, lhs_format, rhs_format, _cref(_config(config))))


def fp8_jit_gemm_workspace_bytes(m, n, k, config) -> int:
    return int(lib().fp8_jit_gemm_workspace_bytes(m, n, k, _cref(_config(config))))


def fp8_jit_gemm_nt(lhs, lhs_format, lhs_scales, rhs, rhs_format, rhs_scales, out, config=None, workspace=None,
                    stream=None):
    """fp8_gemm_nt_fmt through a runtime-specialised kernel (config None:
    the ahead-of-time choice)."""
    lhs_format, rhs_format = _fmt(lhs_format, "lhs_format"), _fmt(rhs_format, "rhs_format")
    lhs, rhs = _codes(lhs, "lhs", lhs_format), _codes(rhs, "rhs", rhs_format)
    lhs_scales, rhs_scales = _f32(lhs_scales, "lhs_scales"), _f32(rhs_scales, "rhs_scales")
    out = _bf16(out, "out")
    m, n, k = _check_gemm_nt(lhs, lhs_scales, rhs, rhs_scales, out, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().fp8_jit_gemm_nt(_p(lhs), lhs_format, _p(lhs_scales), lhs_scales.shape[-1], _p(rhs), rhs_format,
                               _p(rhs_scales), _p(out), m, n, k, _cref(_config(config)), _p(workspace), ws_bytes,
                               _stream(stream))
    _check("fp8_jit_gemm_nt", st)
    return out


def fp8_jit_grouped_gemm_contiguous(lhs, lhs_scales, rhs, rhs_scales, out, m_indices, config=None, stream=None):
    lhs, rhs = _codes(lhs, "lhs"), _codes(rhs, "rhs")
    lhs_scales, rhs_scales = _f32(lhs_scales, "lhs_scales"), _f32(rhs_scales, "rhs_scales")
    out, m_indices = _bf16(out, "out"), _i32t(m_indices, "m_indices")
    M, n, k, G = _check_contiguous(lhs, lhs_scales, rhs, rhs_scales, out, m_indices)
    st = lib().fp8_jit_grouped_gemm_contiguous(_p(lhs), _p(lhs_scales), lhs_scales.shape[-1], _p(rhs),
                                               _p(rhs_scales), _p(out), _p(m_indices), M, n, k, G,
                                               _cref(_config(config)), _stream(stream))
    _check("fp8_jit_grouped_gemm_contiguous", st)
    return out


def fp8_jit_grouped_gemm_masked(lhs, lhs_scales, rhs, rhs_scales, out, masked_m, config=None, stream=None):
    lhs, rhs = _codes(lhs, "lhs"), _codes(rhs, "rhs")
    lhs_scales, rhs_scales = _f32(lhs_scales, "lhs_scales"), _f32(rhs_scales, "rhs_scales")
    out, masked_m = _bf16(out, "out"), _i32t(masked_m, "masked_m")
    G, max_m, n, k = _check_masked(lhs, lhs_scales, rhs, rhs_scales, out, masked_m)
    st = lib().fp8_jit_grouped_gemm_masked(_p(lhs), _p(lhs_scales), lhs_scales.shape[-1], _p(rhs), _p(rhs_scales),
                                           _p(out), _p(masked_m), G, max_m, n, k, _cref(_config(config)),
                                           _stream(stream))
    _check("fp8_jit_grouped_gemm_masked", st)
    return out


def fp8_jit_set_cache_dir(path=None):
    _check("fp8_jit_set_cache_dir", lib().fp8_jit_set_cache_dir(None if path is None else str(path).encode()))


def fp8_jit_get_cache_dir() -> str:
    buf = ctypes.create_string_buffer(4096)
    _check("fp8_jit_get_cache_dir", lib().fp8_jit_get_cache_dir(buf, len(buf)))
    return buf.value.decode()


JIT_STAT_NAMES = ("memory_hits", "disk_hits", "compiles", "rejected_files", "failed_compiles")


def fp8_jit_stats() -> dict:
    arr = (ctypes.c_longlong * len(JIT_STAT_NAMES))()
    _check("fp8_jit_stats", lib().fp8_jit_stats(arr, len(arr)))
    return dict(zip(JIT_STAT_NAMES, list(arr)))


def fp8_grouped_gemm_contiguous(lhs, lhs_scales, rhs, rhs_scales, out, m_indices, stream=None):
    """Contiguous-layout grouped GEMM: lhs [M][k], rhs [G][n][k], m_indices [M]."""
    lhs, rhs = _codes(lhs, "lhs"), _codes(rhs, "rhs")
    lhs_scales, rhs_scales = _f32(lhs_scales, "lhs_scales"), _f32(rhs_scales, "rhs_scales")
    out, m_indices = _bf16(out, "out"), _i32t(m_indices, "m_indices")
    M, n, k, G = _check_contiguous(lhs, lhs_scales, rhs, rhs_scales, out, m_indices)
    st = lib().fp8_grouped_gemm_contiguous(_p(lhs), _p(lhs_scales), lhs_scales.shape[-1], _p(rhs), _p(rhs_scales),
                                           _p(out), _p(m_indices), M, n, k, G, None, 0, _stream(stream))
    _check("fp8_grouped_gemm_contiguous", st)
    return out


def fp8_grouped_gemm_masked(lhs, lhs_scales, rhs, rhs_scales, out, masked_m, stream=None):
    """Masked-layout grouped GEMM: lhs [G][max_m][k], lhs_scales [G][KG][ld],
    rhs [G][n][k], masked_m [G] (device int32)."""
    lhs, rhs = _codes(lhs, "lhs"), _codes(rhs, "rhs")
    lhs_scales, rhs_scales = _f32(lhs_scales, "lhs_scales"), _f32(rhs_scales, "rhs_scales")
    out, masked_m = _bf16(out, "out"), _i32t(masked_m, "masked_m")
    G, max_m, n, k = _check_masked(lhs, lhs_scales, rhs, rhs_scales, out, masked_m)
    st = lib().fp8_grouped_gemm_masked(_p(lhs), _p(lhs_scales), lhs_scales.shape[-1], _p(rhs), _p(rhs_scales),
                                       _p(out), _p(masked_m), G, max_m, n, k, None, 0, _stream(stream))
    _check("fp8_grouped_gemm_masked", st)
    return out


def fp8_cast_per_token_group(x, q, scales, stream=None):
    """x [m][k] float32 or bfloat16 -> q [m][k] codes, scales [KG][ld >= m]."""
    x = _dev(x, "x")
    if x.dtype == torch.float32:
        dt = FP8G_F32
    elif x.dtype == torch.bfloat16:
        dt = FP8G_BF16
    else:
        raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")
    q, scales = _codes(q, "q"), _f32(scales, "scales")
    m, k = _check_cast(x, q, scales)
    st = lib().fp8_cast_per_token_group(_p(x), dt, m, k, _p(q), _p(scales), scales.shape[-1], _stream(stream))
    _check("fp8_cast_per_token_group", st)
    return q, scales


def fp8_cast_per_token_group_fmt(x, q_format, q, scales, stream=None):
    """fp8_cast_per_token_group to q_format (FP8G_E4M3 or FP8G_E5M2)."""
    q_format = _fmt(q_format, "q_format")
    x = _dev(x, "x")
    if x.dtype == torch.float32:
        dt = FP8G_F32
    elif x.dtype == torch.bfloat16:
        dt = FP8G_BF16
    else:
        raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")
    q, scales = _codes(q, "q", q_format), _f32(scales, "scales")
    m, k = _check_cast(x, q, scales)
    st = lib().fp8_cast_per_token_group_fmt(_p(x), dt, q_format, m, k, _p(q), _p(scales), scales.shape[-1],
                                            _stream(stream))
    _check("fp8_cast_per_token_group_fmt", st)
    return q, scales


def fp8_cast_per_block_fmt(w, q_format, q, scales, stream=None):
    """fp8_cast_per_block to q_format (FP8G_E4M3 or FP8G_E5M2)."""
    q_format = _fmt(q_format, "q_format")
    w = _f32(w, "w")
    q, scales = _codes(q, "q", q_format), _f32(scales, "scales")
    n, k = _check_block_cast(w, q, scales)
    st = lib().fp8_cast_per_block_fmt(_p(w), q_format, n, k, _p(q), _p(scales), _stream(stream))
    _check("fp8_cast_per_block_fmt", st)
    return q, scales


def fp8_cast_per_block(w, q, scales, stream=None):
    """w [n][k] float32 -> q [n][k] codes, scales [NB][KG] (128 x 128 blocks)."""
    w = _f32(w, "w")
    q, scales = _codes(q, "q"), _f32(scales, "scales")
    n, k = _check_block_cast(w, q, scales)
    st = lib().fp8_cast_per_block(_p(w), n, k, _p(q), _p(scales), _stream(stream))
    _check("fp8_cast_per_block", st)
    return q, scales


def fp8_gemm_workspace_bytes(m, n, k, num_groups=1) -> int:
    return int(lib().fp8_gemm_workspace_bytes(int(m), int(n), int(k), int(num_groups)))


def fp8_gemm_describe(m: int, n: int, k: int) -> str:
    """The dense configuration fp8_gemm_nt picks for (m, n, k), as text
    (host only; launches nothing)."""
    buf = ctypes.create_string_buffer(256)
    st = lib().fp8_gemm_describe(m, n, k, buf, len(buf))
    _check("fp8_gemm_describe", st)
    return buf.value.decode()


def fp8_gemm_schedule(mode, m, n, k, num_groups=0, group_data=None):
    """Host only: the work unit each workgroup of the GEMM call takes, as an
    int32 numpy array [workgroups][6] of (taken, group, first row, rows,
    column tile, split) in launch order.  group_data is a host int32 array
    (contiguous: m_indices; masked: masked_m)."""
    import numpy as np
    gd = None if group_data is None else np.ascontiguousarray(group_data, dtype=np.int32)
    gp = None if gd is None else gd.ctypes.data_as(ctypes.c_void_p)
    count = lib().fp8_gemm_schedule(mode, m, n, k, num_groups, gp, None, 0)
    _check("fp8_gemm_schedule", min(count, 0))
    units = np.zeros((max(count, 1), 6), np.int32)
    got = lib().fp8_gemm_schedule(mode, m, n, k, num_groups, gp, units.ctypes.data_as(ctypes.c_void_p), count)
    _check("fp8_gemm_schedule", min(got, 0))
    assert got == count
    return units[:count]


def fp8_set_num_cus(num_cus: int) -> int:
    return int(lib().fp8_set_num_cus(int(num_cus)))


def fp8_get_num_cus() -> int:
    return int(lib().fp8_get_num_cus())


def fp8_status_string(status: int) -> str:
    return status_string(status)


# ---- MoE layout steps ----------------------------------------------------------
def fp8_moe_contiguous_rows(num_tokens: int, num_groups: int) -> int:
    return int(lib().fp8_moe_contiguous_rows(int(num_tokens), int(num_groups)))


def fp8_moe_layout_workspace_bytes(num_tokens: int, num_groups: int) -> int:
    return int(lib().fp8_moe_layout_workspace_bytes(int(num_tokens), int(num_groups)))


def _workspace(nbytes, device):
    return torch.empty(max(1, (nbytes + 3) // 4), dtype=torch.int32, device=device)


def fp8_moe_layout_contiguous(expert_idx, num_groups, m_rows=None, workspace=None, stream=None):
    """Contiguous (prefill) layout of a routing.  Returns (counts [G],
    offsets [G+1], dst_row [T], m_indices [m_rows]) as int32 device tensors."""
    expert_idx = _i32t(expert_idx, "expert_idx")
    _want_dim(expert_idx, "expert_idx", 1)
    T = expert_idx.numel()
    G = int(num_groups)
    if m_rows is None:
        m_rows = fp8_moe_contiguous_rows(T, G)
    dev = expert_idx.device
    if workspace is not None:
        _dev(workspace, "workspace")
        _same_device(expert_idx=expert_idx, workspace=workspace)
    counts = torch.empty(G, dtype=torch.int32, device=dev)
    offsets = torch.empty(G + 1, dtype=torch.int32, device=dev)
    dst = torch.empty(max(T, 1), dtype=torch.int32, device=dev)[:T]
    m_indices = torch.empty(max(int(m_rows), 1), dtype=torch.int32, device=dev)[:int(m_rows)]
    if workspace is None:
        workspace = _workspace(fp8_moe_layout_workspace_bytes(T, G), dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().fp8_moe_layout_contiguous(_p(expert_idx), T, G, _p(counts), _p(offsets), _p(dst), _p(m_indices),
                                         int(m_rows), _p(workspace), ws_bytes, _stream(stream))
    _check("fp8_moe_layout_contiguous", st)
    return counts, offsets, dst, m_indices


def fp8_moe_layout_masked(expert_idx, num_groups, max_m, workspace=None, stream=None):
    """Masked (decode) layout of a routing.  Returns (counts [G], dst_row [T],
    masked_m [G]) as int32 device tensors."""
    expert_idx = _i32t(expert_idx, "expert_idx")
    _want_dim(expert_idx, "expert_idx", 1)
    T = expert_idx.numel()
    G = int(num_groups)
    dev = expert_idx.device
    if workspace is not None:
        _dev(workspace, "workspace")
        _same_device(expert_idx=expert_idx, workspace=workspace)
    counts = torch.empty(G, dtype=torch.int32, device=dev)
    masked_m = torch.empty(G, dtype=torch.int32, device=dev)
    dst = torch.empty(max(T, 1), dtype=torch.int32, device=dev)[:T]
    if workspace is None:
        workspace = _workspace(fp8_moe_layout_workspace_bytes(T, G), dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().fp8_moe_layout_masked(_p(expert_idx), T, G, int(max_m), _p(counts), _p(dst), _p(masked_m),
                                     _p(workspace), ws_bytes, _stream(stream))
    _check("fp8_moe_layout_masked", st)
    return counts, dst, masked_m


def fp8_moe_scatter_rows(q, scales, dst_row, q_out, scales_out, rows_per_group=None, stream=None):
    """q [T][k] codes and scales [KG][ld >= T] to their laid-out rows.
    Contiguous: q_out [M][k], scales_out [KG][ld >= M].  Masked: q_out
    [G][max_m][k], scales_out [G][KG][ld >= max_m] (rows_per_group = max_m)."""
    q, q_out = _codes(q, "q"), _codes(q_out, "q_out")
    scales, scales_out = _f32(scales, "scales"), _f32(scales_out, "scales_out")
    dst_row = _i32t(dst_row, "dst_row")
    _want_dim(q, "q", 2)
    T, k = q.shape
    _want_scales_mn(scales, "scales", (_kg(k),), T)
    _want(dst_row, "dst_row", (T,))
    if q_out.dim() not in (2, 3) or q_out.shape[-1] != k:
        raise ValueError(f"q_out has shape {tuple(q_out.shape)}, expected (rows, {k}) or (G, max_m, {k})")
    out_rows = q_out.numel() // k if k else 0
    if rows_per_group is None:
        rows_per_group = q_out.shape[-2] if q_out.dim() == 3 else out_rows
    rows_per_group = int(rows_per_group)
    # scales_out: one MN-major [KG][ld >= rows_per_group] block per group of rows
    groups = -(-out_rows // rows_per_group) if rows_per_group > 0 else 0
    if (scales_out.dim() < 2 or scales_out.shape[-2] != _kg(k) or scales_out.shape[-1] < rows_per_group
            or scales_out.numel() < groups * _kg(k) * scales_out.shape[-1]):
        raise ValueError(f"scales_out has shape {tuple(scales_out.shape)}, expected {groups} block(s) of "
                         f"({_kg(k)}, ld >= {rows_per_group})")
    _same_device(q=q, scales=scales, dst_row=dst_row, q_out=q_out, scales_out=scales_out)
    st = lib().fp8_moe_scatter_rows(_p(q), _p(scales), scales.shape[-1], T, k, _p(dst_row), int(rows_per_group),
                                    int(out_rows), _p(q_out), _p(scales_out), scales_out.shape[-1], _stream(stream))
    _check("fp8_moe_scatter_rows", st)
    return q_out, scales_out


def fp8_moe_gather_rows(y, dst_row, out, stream=None):
    """out[t] = y[dst_row[t]] (bfloat16 rows), zeros where dst_row[t] < 0."""
    y, out = _bf16(y, "y"), _bf16(out, "out")
    dst_row = _i32t(dst_row, "dst_row")
    _want_dim(dst_row, "dst_row", 1)
    _want_dim(out, "out", 2)
    n = out.shape[-1]
    _want(out, "out", (dst_row.numel(), n))
    if y.dim() < 1 or y.shape[-1] != n:
        raise ValueError(f"y has shape {tuple(y.shape)}, expected rows of {n} outputs")
    y_rows = y.numel() // n if n else 0
    _same_device(y=y, dst_row=dst_row, out=out)
    st = lib().fp8_moe_gather_rows(_p(y), n, y_rows, _p(dst_row), dst_row.numel(), _p(out), _stream(stream))
    _check("fp8_moe_gather_rows", st)
    return out
