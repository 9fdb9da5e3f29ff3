"""ctypes binding of libarrms.so (include/arrms.h), same names as the C ABI.

Argument marshalling only: tensors become device pointers, the stream becomes
the HIP stream handle, and a negative status becomes an ``ArrmsError``. Every
step of the epilogue runs in the library's HIP kernels. Importing this module
loads the library and raises ``ImportError`` when it has not been built
(``python -m all_reduce_residual_rank_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

# PyTorch-ROCm bundles its own HIP runtime (soname libamdhip64.so.7). Loading
# torch first makes libarrms.so bind to that same runtime; loading the library
# first would pull in /opt/rocm's runtime as a second copy, whose launches
# reject torch's stream handles.
try:
    import torch  # noqa: F401
except ImportError:  # pragma: no cover - torch is the memory/stream provider here
    torch = None

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libarrms.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with "
                      "`python -m all_reduce_residual_rank_amd.build` (hipcc, gfx950)")
_lib = ctypes.CDLL(_LIB_PATH)

# constants of include/arrms.h
OK = 0
ERR_INVALID = -1
ERR_UNSUPPORTED = -2
ERR_NO_STAGING = -3
ERR_HIP = -4
DTYPE_BF16, DTYPE_FP16, DTYPE_FP32 = 0, 1, 2
GEMMA = 4
FP8 = 8
FORCE_ONE_STAGE = 16
FORCE_TWO_STAGE = 32
EXACT_ONLY = 64
MAX_RANKS = 8
MAX_HIDDEN = 16384
MAX_ROW_BYTES = 65536
DEFAULT_STAGING_BYTES = 16 << 20
PATH_NONE, PATH_ONE_STAGE, PATH_TWO_STAGE = 0, 1, 2

QUANT_FP8_TOKEN, QUANT_FP8_GROUP, QUANT_MXFP4 = 1, 2, 3
FP8_GROUP_SIZE = 128
MX_BLOCK = 32

NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTS = ("arrms_fused", "arrms_fused_noalloc", "arrms_fused_strided", "arrms_fused_quant", "arrms_allreduce_sum",
           "arrms_fused_config", "arrms_query_launch", "arrms_plan_launch",
           "arrms_reserve_staging", "arrms_release_staging", "arrms_staging_bytes", "arrms_query_path",
           "arrms_status_string")

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_ll = ctypes.c_longlong
_lib.arrms_fused.argtypes = [ctypes.POINTER(_vp), _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _f, _i, _vp]
_lib.arrms_fused.restype = _i
_lib.arrms_fused_noalloc.argtypes = [ctypes.POINTER(_vp), _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _f, _i, _vp]
_lib.arrms_fused_noalloc.restype = _i
_lib.arrms_fused_strided.argtypes = [ctypes.POINTER(_vp), _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i,
                                     _ll, _ll, _ll, _ll, _ll, _f, _i, _vp]
_lib.arrms_fused_strided.restype = _i
_lib.arrms_fused_quant.argtypes = [ctypes.POINTER(_vp), _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _f, _i,
                                   _i, _vp]
_lib.arrms_fused_quant.restype = _i
_lib.arrms_allreduce_sum.argtypes = [ctypes.POINTER(_vp), _i, _vp, _ll, _i, _vp]
_lib.arrms_allreduce_sum.restype = _i
_lib.arrms_fused_config.argtypes = [ctypes.POINTER(_vp), _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _f, _i,
                                    _i, _i, _i, _i, _i, _vp]
_lib.arrms_fused_config.restype = _i
_lib.arrms_query_launch.argtypes = [_i, _i, _i, _i, _i, _i, ctypes.POINTER(_i)]
_lib.arrms_query_launch.restype = _i
_lib.arrms_plan_launch.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i, ctypes.POINTER(_i)]
_lib.arrms_plan_launch.restype = _i
_lib.arrms_reserve_staging.argtypes = [_sz]
_lib.arrms_reserve_staging.restype = _i
_lib.arrms_release_staging.argtypes = []
_lib.arrms_release_staging.restype = _i
_lib.arrms_staging_bytes.argtypes = []
_lib.arrms_staging_bytes.restype = _sz
_lib.arrms_query_path.argtypes = [_i, _i, _i, _i]
_lib.arrms_query_path.restype = _i
_lib.arrms_status_string.argtypes = [_i]
_lib.arrms_status_string.restype = ctypes.c_char_p

LIB_PATH = _LIB_PATH


class ArrmsError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({arrms_status_string(status)})")
        self.status = status


def arrms_status_string(status: int) -> str:
    return _lib.arrms_status_string(int(status)).decode()


def _addr(t) -> int | None:
    """Device address of a tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


_T_BY_CODE = {DTYPE_BF16: "bfloat16", DTYPE_FP16: "float16", DTYPE_FP32: "float32"}


def _check(t, name: str, *, dtype=None, numel: int = 0, nbytes: int = 0, contiguous: bool = True,
           device=None) -> None:
    """Host-side check of one tensor argument before its address goes to the C
    ABI: a GPU tensor (on `device` when given), of `dtype` (a torch dtype name,
    or None for any), contiguous when asked, holding at least `numel` elements
    or `nbytes` bytes from its first element on. Ints (raw addresses) and None
    pass unchecked. Raises ValueError."""
    if t is None or isinstance(t, int):
        return
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other operands on {device}")
    if dtype is not None and str(t.dtype) != f"torch.{dtype}":
        raise ValueError(f"{name} must be {dtype} for these flags (got {t.dtype})")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (use arrms_fused_strided for padded rows)")
    have = t.untyped_storage().nbytes() - t.storage_offset() * t.element_size()
    need = max(numel * t.element_size(), nbytes)
    if have < need:
        raise ValueError(f"{name} holds {have} bytes from its first element, the call needs {need}")


def _check_fused(rank_in, residual, weight, out, residual_out, fp8_out, fp8_scale, M, H, flags,
                 q_bytes=None, s_bytes=None, strides=None):
    """Checks of the fused entry points' tensors against M, H and the flags.
    strides: (ld_in, ld_residual, ld_out, ld_residual_out, ld_fp8) for the
    strided form (rows may be padded), else None (contiguous [M][H])."""
    if M < 0 or H < 1:
        return  # the C ABI rejects these sizes itself
    dt = _T_BY_CODE.get(flags & 3)
    dev = residual.device if hasattr(residual, "device") else None

    def span(ld):
        return 0 if M == 0 else (M - 1) * ld + H

    ld = strides or (H, H, H, H, H)
    contig = strides is None
    for r, x in enumerate(rank_in):
        _check(x, f"rank_in[{r}]", dtype=dt, numel=span(ld[0]), contiguous=contig, device=dev)
    _check(residual, "residual", dtype=dt, numel=span(ld[1]), contiguous=contig)
    _check(weight, "weight", dtype=dt, numel=H, device=dev)
    _check(out, "out", dtype=dt, numel=span(ld[2]), contiguous=contig, device=dev)
    _check(residual_out, "residual_out", dtype=dt, numel=span(ld[3]), contiguous=contig, device=dev)
    if flags & FP8 or q_bytes is not None:
        qb = (M * H if q_bytes is None else q_bytes) if contig else (0 if M == 0 else (M - 1) * ld[4] + H)
        sb = M * 4 if s_bytes is None else s_bytes
        _check(fp8_out, "fp8_out", nbytes=qb, contiguous=contig, device=dev)
        _check(fp8_scale, "fp8_scale", nbytes=sb, device=dev)


def _stream_handle(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def arrms_fused_raw(rank_in, R, residual, weight, out, residual_out, fp8_out, fp8_scale,
                    M, H, eps, flags, stream) -> int:
    """The C call with addresses as ints; returns the status unchanged."""
    ptrs = (_vp * max(len(rank_in), 1))(*[_addr(p) for p in rank_in])
    return _lib.arrms_fused(ptrs, int(R), _addr(residual), _addr(weight), _addr(out),
                            _addr(residual_out), _addr(fp8_out), _addr(fp8_scale), int(M), int(H),
                            float(eps), int(flags), stream)


def arrms_fused_config_raw(rank_in, R, residual, weight, out, residual_out, fp8_out, fp8_scale,
                           M, H, eps, flags, ppt, tpr, rows_per_block, blocks, stream,
                           load_window=0) -> int:
    """arrms_fused_config with addresses as ints; returns the status unchanged."""
    ptrs = (_vp * max(len(rank_in), 1))(*[_addr(p) for p in rank_in])
    return _lib.arrms_fused_config(ptrs, int(R), _addr(residual), _addr(weight), _addr(out),
                                   _addr(residual_out), _addr(fp8_out), _addr(fp8_scale), int(M),
                                   int(H), float(eps), int(flags), int(ppt), int(tpr),
                                   int(rows_per_block), int(blocks), int(load_window), stream)


def arrms_fused_config(rank_in, residual, weight, out, residual_out, fp8_out=None, fp8_scale=None, *,
                       eps: float, flags: int, ppt: int = 0, tpr: int = 0, rows_per_block: int = 0,
                       blocks: int = 0, load_window: int = 0, M: int | None = None,
                       H: int | None = None, stream=None) -> None:
    """arrms_fused with an explicit row-kernel launch shape (0 = automatic)."""
    if M is None or H is None:
        M, H = residual.shape[-2], residual.shape[-1]
    _check_fused(rank_in, residual, weight, out, residual_out, fp8_out, fp8_scale, M, H, flags)
    rc = arrms_fused_config_raw(rank_in, len(rank_in), residual, weight, out, residual_out, fp8_out,
                                fp8_scale, M, H, eps, flags, ppt, tpr, rows_per_block, blocks,
                                _stream_handle(stream), load_window=load_window)
    if rc != OK:
        raise ArrmsError(rc, "arrms_fused_config")


def arrms_fused(rank_in, residual, weight, out, residual_out, fp8_out=None, fp8_scale=None, *,
                eps: float, flags: int, M: int | None = None, H: int | None = None, stream=None) -> None:
    """Enqueue the fused epilogue on ``stream`` (default: torch's current stream).

    rank_in: list of R device tensors [M][H] (or addresses); the other arguments
    as in include/arrms.h. M and H default to the residual's shape.
    """
    if M is None or H is None:
        M, H = residual.shape[-2], residual.shape[-1]
    _check_fused(rank_in, residual, weight, out, residual_out, fp8_out, fp8_scale, M, H, flags)
    st = _stream_handle(stream)
    rc = arrms_fused_raw(rank_in, len(rank_in), residual, weight, out, residual_out, fp8_out,
                         fp8_scale, M, H, eps, flags, st)
    if rc != OK:
        raise ArrmsError(rc, "arrms_fused")


def arrms_fused_noalloc_raw(rank_in, R, residual, weight, out, residual_out, fp8_out, fp8_scale,
                            M, H, eps, flags, stream) -> int:
    """arrms_fused_noalloc with addresses as ints; returns the status unchanged."""
    ptrs = (_vp * max(len(rank_in), 1))(*[_addr(p) for p in rank_in])
    return _lib.arrms_fused_noalloc(ptrs, int(R), _addr(residual), _addr(weight), _addr(out),
                                    _addr(residual_out), _addr(fp8_out), _addr(fp8_scale), int(M), int(H),
                                    float(eps), int(flags), stream)


def arrms_fused_noalloc(rank_in, residual, weight, out, residual_out, fp8_out=None, fp8_scale=None, *,
                        eps: float, flags: int, M: int | None = None, H: int | None = None,
                        stream=None) -> None:
    """arrms_fused that never allocates: the two-stage path stages through the
    library's fixed per-GPU region (calls on one GPU share it)."""
    if M is None or H is None:
        M, H = residual.shape[-2], residual.shape[-1]
    _check_fused(rank_in, residual, weight, out, residual_out, fp8_out, fp8_scale, M, H, flags)
    rc = arrms_fused_noalloc_raw(rank_in, len(rank_in), residual, weight, out, residual_out, fp8_out,
                                 fp8_scale, M, H, eps, flags, _stream_handle(stream))
    if rc != OK:
        raise ArrmsError(rc, "arrms_fused_noalloc")


def arrms_fused_strided_raw(rank_in, R, residual, weight, out, residual_out, fp8_out, fp8_scale,
                            M, H, ld_in, ld_residual, ld_out, ld_residual_out, ld_fp8, eps, flags,
                            stream) -> int:
    """arrms_fused_strided with addresses as ints; returns the status unchanged."""
    ptrs = (_vp * max(len(rank_in), 1))(*[_addr(p) for p in rank_in])
    return _lib.arrms_fused_strided(ptrs, int(R), _addr(residual), _addr(weight), _addr(out),
                                    _addr(residual_out), _addr(fp8_out), _addr(fp8_scale), int(M),
                                    int(H), int(ld_in), int(ld_residual), int(ld_out),
                                    int(ld_residual_out), int(ld_fp8), float(eps), int(flags), stream)


def _row_stride(t, default: int) -> int:
    if t is None or isinstance(t, int):
        return default
    if t.dim() < 2 or t.stride(-1) != 1:
        raise ValueError("strided rows need a unit stride along the last dimension")
    return int(t.stride(-2))


def arrms_fused_strided(rank_in, residual, weight, out, residual_out, fp8_out=None, fp8_scale=None, *,
                        eps: float, flags: int, M: int | None = None, H: int | None = None,
                        ld_in: int | None = None, ld_residual: int | None = None,
                        ld_out: int | None = None, ld_residual_out: int | None = None,
                        ld_fp8: int | None = None, stream=None) -> None:
    """arrms_fused over row-strided matrices (for instance column slices of
    wider tensors). Strides default to each tensor's own row stride."""
    if M is None or H is None:
        M, H = residual.shape[-2], residual.shape[-1]
    if ld_in is None:
        strides = {_row_stride(t, H) for t in rank_in}
        if len(strides) != 1:
            raise ValueError("all rank inputs must share one row stride")
        ld_in = strides.pop()
    ld_residual = _row_stride(residual, H) if ld_residual is None else ld_residual
    ld_out = _row_stride(out, H) if ld_out is None else ld_out
    ld_residual_out = _row_stride(residual_out, H) if ld_residual_out is None else ld_residual_out
    ld_fp8 = _row_stride(fp8_out, H) if ld_fp8 is None else ld_fp8
    _check_fused(rank_in, residual, weight, out, residual_out, fp8_out, fp8_scale, M, H, flags,
                 strides=(ld_in, ld_residual, ld_out, ld_residual_out, ld_fp8))
    rc = arrms_fused_strided_raw(rank_in, len(rank_in), residual, weight, out, residual_out, fp8_out,
                                 fp8_scale, M, H, ld_in, ld_residual, ld_out, ld_residual_out, ld_fp8,
                                 eps, flags, _stream_handle(stream))
    if rc != OK:
        raise ArrmsError(rc, "arrms_fused_strided")


def arrms_fused_quant_raw(rank_in, R, residual, weight, out, residual_out, q_out, q_scale, M, H, eps,
                          flags, quant, stream) -> int:
    """arrms_fused_quant with addresses as ints; returns the status unchanged."""
    ptrs = (_vp * max(len(rank_in), 1))(*[_addr(p) for p in rank_in])
    return _lib.arrms_fused_quant(ptrs, int(R), _addr(residual), _addr(weight), _addr(out),
                                  _addr(residual_out), _addr(q_out), _addr(q_scale), int(M), int(H),
                                  float(eps), int(flags), int(quant), stream)


def arrms_fused_quant(rank_in, residual, weight, out, residual_out, q_out, q_scale, *, eps: float,
                      flags: int, quant: int, M: int | None = None, H: int | None = None,
                      stream=None) -> None:
    """The fused epilogue with a quantised output (QUANT_FP8_TOKEN, QUANT_FP8_GROUP
    or QUANT_MXFP4); ``out`` is the optional T mirror."""
    if M is None or H is None:
        M, H = residual.shape[-2], residual.shape[-1]
    if quant == QUANT_FP8_GROUP:
        qb, sb = M * H, M * (H // FP8_GROUP_SIZE) * 4
    elif quant == QUANT_MXFP4:
        qb, sb = M * H // 2, M * (H // MX_BLOCK)
    else:
        qb, sb = M * H, M * 4
    _check_fused(rank_in, residual, weight, out, residual_out, q_out, q_scale, M, H, flags,
                 q_bytes=qb, s_bytes=sb)
    rc = arrms_fused_quant_raw(rank_in, len(rank_in), residual, weight, out, residual_out, q_out, q_scale,
                               M, H, eps, flags, quant, _stream_handle(stream))
    if rc != OK:
        raise ArrmsError(rc, "arrms_fused_quant")


def arrms_allreduce_sum_raw(rank_in, R, out, n, flags, stream) -> int:
    """arrms_allreduce_sum with addresses as ints; returns the status unchanged."""
    ptrs = (_vp * max(len(rank_in), 1))(*[_addr(p) for p in rank_in])
    return _lib.arrms_allreduce_sum(ptrs, int(R), _addr(out), int(n), int(flags), stream)


def arrms_allreduce_sum(rank_in, out, *, flags: int, n: int | None = None, stream=None) -> None:
    """Enqueue the rank-ordered sum of the R rank tensors into ``out``
    (contiguous tensors of n elements; n defaults to out.numel())."""
    if n is None:
        n = out.numel()
    dt = _T_BY_CODE.get(flags & 3) if not (flags & ~3) else None
    dev = out.device if hasattr(out, "device") else None
    for r, x in enumerate(rank_in):
        _check(x, f"rank_in[{r}]", dtype=dt, numel=n, device=dev)
    _check(out, "out", dtype=dt, numel=n)
    rc = arrms_allreduce_sum_raw(rank_in, len(rank_in), out, n, flags, _stream_handle(stream))
    if rc != OK:
        raise ArrmsError(rc, "arrms_allreduce_sum")


LAUNCH_INFO = 8
LAUNCH_FIELDS = ("path", "ppt", "tpr", "rpb", "window", "cap16", "blocks_per_cu", "cus")


def arrms_query_launch(M: int, H: int, R: int, flags: int, quant: int = 0, mirror: bool = False) -> dict:
    """The row-kernel launch arrms_fused makes for these sizes on the current
    device (arrms_tuning.h), as a dict of LAUNCH_FIELDS."""
    info = (_i * LAUNCH_INFO)()
    rc = _lib.arrms_query_launch(int(M), int(H), int(R), int(flags), int(quant), int(bool(mirror)), info)
    if rc != OK:
        raise ArrmsError(rc, "arrms_query_launch")
    return dict(zip(LAUNCH_FIELDS, list(info)))


def arrms_plan_launch(M: int, H: int, R: int, flags: int, quant: int, mirror: bool, blocks_per_cu: int,
                      cus: int) -> dict:
    """The same launch from given device facts (pure host)."""
    info = (_i * LAUNCH_INFO)()
    rc = _lib.arrms_plan_launch(int(M), int(H), int(R), int(flags), int(quant), int(bool(mirror)),
                                int(blocks_per_cu), int(cus), info)
    if rc != OK:
        raise ArrmsError(rc, "arrms_plan_launch")
    return dict(zip(LAUNCH_FIELDS, list(info)))


def arrms_reserve_staging(nbytes: int = 0) -> None:
    rc = _lib.arrms_reserve_staging(int(nbytes))
    if rc != OK:
        raise ArrmsError(rc, "arrms_reserve_staging")


def arrms_release_staging() -> None:
    rc = _lib.arrms_release_staging()
    if rc != OK:
        raise ArrmsError(rc, "arrms_release_staging")


def arrms_staging_bytes() -> int:
    return int(_lib.arrms_staging_bytes())


def arrms_query_path(M: int, H: int, R: int, flags: int) -> int:
    return int(_lib.arrms_query_path(int(M), int(H), int(R), int(flags)))
