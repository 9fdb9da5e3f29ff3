"""CPU oracle for the fused rank-sum + residual-add + RMSNorm (+ per-token FP8) epilogue.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It is a ctypes
wrapper around ``oracle.c`` (plain single-threaded C, compiled with gcc and
``-ffp-contract=off``), which defines what the fused epilogue computes; it
shares no code with the HIP library and never loads it.

Arrays cross the boundary as raw storage bits: ``numpy.uint16`` for bf16 and
fp16, ``numpy.float32`` for fp32, ``numpy.uint8`` for FP8 E4M3 codes.

Every function here is pinned by ``tests/test_oracle_*.py`` against the
format definitions, closed forms, brute force in exact rational arithmetic
and independent library casts (numpy / torch); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# flag bits as the oracle reads them (dtype in bits 0-1, gemma_norm, and at
# most one quantised output: per-token FP8, per-group FP8, MXFP4)
BF16, FP16, FP32 = 0, 1, 2
GEMMA = 4
FP8 = 8
FP8_GROUP = 16
MXFP4 = 32
GROUP = 128       # per-group FP8: columns per scale
MX_BLOCK = 32     # MXFP4: columns per E8M0 scale
QUANT = FP8 | FP8_GROUP | MXFP4

_lib = None


def build() -> str:
    """Compile oracle.c into liboracle.so next to it (always recompiles)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
           "-Wall", "-Wextra", "-fPIC", "-shared", _SRC, "-o", _LIB_PATH, "-lm"]
    subprocess.check_call(cmd)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    stale = (not os.path.exists(_LIB_PATH)
             or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC))
    if stale:
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.oracle_fused_rows.argtypes = [ctypes.POINTER(vp), i, vp, vp, vp, vp, vp, vp,
                                      i, i, f, i, i, i, vp]
    lib.oracle_fused_rows.restype = i
    lib.oracle_quant_rows.argtypes = [vp, i, i, i, vp, vp]
    lib.oracle_quant_rows.restype = i
    lib.oracle_rank_sum.argtypes = [ctypes.POINTER(vp), i, vp, ctypes.c_size_t, i]
    lib.oracle_rank_sum.restype = i
    sz = ctypes.c_size_t
    for name in ("orc_bf16_from_double_n", "orc_fp16_from_double_n", "orc_e4m3_from_float_n",
                 "orc_e2m1_from_float_n"):
        getattr(lib, name).argtypes = [vp, vp, sz]
        getattr(lib, name).restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def storage_dtype(dt: int):
    return np.float32 if dt == FP32 else np.uint16


def fused(xs, residual, weight, eps: float, flags: int, *, want_out: bool = True,
          rows: tuple[int, int] | None = None, residual_out_inplace: bool = False):
    """Run the oracle on host arrays.

    xs: list of R arrays [M][H] (storage bits of T); residual [M][H]; weight [H].
    flags: dtype | GEMMA | at most one of FP8, FP8_GROUP, MXFP4. With a
    quantised output, ``want_out`` controls the T mirror. 'fp8' holds the
    codes ([M][H] E4M3, or [M][H/2] packed E2M1 for MXFP4) and 'scale' the
    scales ([M] or [M][H/128] fp32, or [M][H/32] E8M0 bytes).
    rows: optional (begin, end) row range; rows outside it are left zero.
    residual_out_inplace: write residual_out into ``residual`` itself.
    Returns a dict with 'out', 'residual_out', 'fp8', 'scale' (absent ones None).
    """
    lib = _load()
    dt = flags & 3
    sdt = storage_dtype(dt)
    xs = [np.ascontiguousarray(x, dtype=sdt) for x in xs]
    M, H = xs[0].shape
    for x in xs:
        assert x.shape == (M, H)
    if residual_out_inplace:
        assert residual.dtype == sdt and residual.flags.c_contiguous
    else:
        residual = np.ascontiguousarray(residual, dtype=sdt)
    weight = np.ascontiguousarray(weight, dtype=sdt).reshape(H)
    b, e = rows if rows is not None else (0, M)
    quant = flags & QUANT
    out = np.zeros((M, H), dtype=sdt) if want_out else None
    res_out = residual if residual_out_inplace else np.zeros((M, H), dtype=sdt)
    q = sc = None
    if quant == FP8:
        q, sc = np.zeros((M, H), dtype=np.uint8), np.zeros((M,), dtype=np.float32)
    elif quant == FP8_GROUP:
        q, sc = np.zeros((M, H), dtype=np.uint8), np.zeros((M, H // GROUP), dtype=np.float32)
    elif quant == MXFP4:
        q, sc = np.zeros((M, H // 2), dtype=np.uint8), np.zeros((M, H // MX_BLOCK), dtype=np.uint8)
    ptrs = (ctypes.c_void_p * len(xs))(*[x.ctypes.data for x in xs])
    scratch = np.empty((H,), dtype=np.float32)
    rc = lib.oracle_fused_rows(ptrs, len(xs), _ptr(residual), _ptr(weight), _ptr(out),
                               _ptr(res_out), _ptr(q), _ptr(sc), M, H, float(eps), int(flags),
                               int(b), int(e), _ptr(scratch))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
    return {"out": out, "residual_out": res_out, "fp8": q, "scale": sc}


def rank_sum(xs, dt: int) -> np.ndarray:
    """Step O1 alone: the rank-ordered sum of the R arrays (storage bits of T,
    any equal shapes), rounded to T. Returns an array of the same shape."""
    lib = _load()
    sdt = storage_dtype(dt)
    xs = [np.ascontiguousarray(x, dtype=sdt) for x in xs]
    shape = xs[0].shape
    for x in xs:
        assert x.shape == shape
    out = np.zeros(shape, dtype=sdt)
    ptrs = (ctypes.c_void_p * len(xs))(*[x.ctypes.data for x in xs])
    rc = lib.oracle_rank_sum(ptrs, len(xs), _ptr(out), int(out.size), int(dt))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
    return out


def quant(y: np.ndarray, dt: int):
    """Step O5 alone on T rows y [M][H]: returns (fp8 codes [M][H], scales [M])."""
    lib = _load()
    y = np.ascontiguousarray(y, dtype=np.uint16)
    M, H = y.shape
    q = np.zeros((M, H), dtype=np.uint8)
    sc = np.zeros((M,), dtype=np.float32)
    rc = lib.oracle_quant_rows(_ptr(y), int(dt), M, H, _ptr(q), _ptr(sc))
    if rc != 0:
        raise ValueError("oracle_quant_rows: bad dtype")
    return q, sc


def bf16_from_double(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64).ravel()
    o = np.empty(v.shape, dtype=np.uint16)
    _load().orc_bf16_from_double_n(_ptr(v), _ptr(o), v.size)
    return o


def fp16_from_double(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64).ravel()
    o = np.empty(v.shape, dtype=np.uint16)
    _load().orc_fp16_from_double_n(_ptr(v), _ptr(o), v.size)
    return o


def e2m1_from_float(v) -> np.ndarray:
    """E2M1 codes (low nibble) of fp32 values, RNE, saturating to +-6."""
    lib = _load()
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.zeros(v.shape, dtype=np.uint8)
    lib.orc_e2m1_from_float_n(_ptr(v), _ptr(out), v.size)
    return out


def e4m3_from_float(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    o = np.empty(v.shape, dtype=np.uint8)
    _load().orc_e4m3_from_float_n(_ptr(v), _ptr(o), v.size)
    return o
