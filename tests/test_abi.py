"""The C ABI on the host (no GPU): the library loads, exports what include/arrms.h
declares, and rejects bad arguments before touching any device.

Only argument checks are exercised here: every call below returns from the
host-side validation (or from M == 0) and launches nothing. Device pointers are
fake, aligned addresses that are never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import pytest

from all_reduce_residual_rank_amd import arrms

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]

BASE = 1 << 40          # fake device addresses, far apart
STRIDE = 1 << 32


def _headers_text():
    return "\n".join(open(h).read() for h in HEADERS)


def declared_functions():
    text = _headers_text()
    return sorted(set(re.findall(r"ARRMS_API\s+[\w\s\*]*?\b(arrms_\w+)\s*\(", text)))


def header_constants():
    text = _headers_text()
    out = {}
    for name, val in re.findall(r"#define\s+ARRMS_(\w+)\s+\(?(-?\d+)u?\)?\s", text):
        out[name] = int(val)
    return out


def test_exports_match_header():
    decl = declared_functions()
    assert decl == sorted(arrms.EXPORTS)
    nm = subprocess.run(["nm", "-D", "--defined-only", arrms.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(arrms_\w+)$", nm, re.M))
    assert exported == set(decl)
    lib = ctypes.CDLL(arrms.LIB_PATH)
    for name in decl:
        assert getattr(lib, name) is not None


def test_binding_constants_match_header():
    c = header_constants()
    for name in ("OK", "ERR_INVALID", "ERR_UNSUPPORTED", "ERR_NO_STAGING", "ERR_HIP", "DTYPE_BF16",
                 "DTYPE_FP16", "DTYPE_FP32", "GEMMA", "FP8", "FORCE_ONE_STAGE", "FORCE_TWO_STAGE",
                 "EXACT_ONLY", "MAX_RANKS", "MAX_HIDDEN", "MAX_ROW_BYTES", "PATH_NONE", "PATH_ONE_STAGE",
                 "PATH_TWO_STAGE", "QUANT_FP8_TOKEN", "QUANT_FP8_GROUP", "QUANT_MXFP4",
                 "FP8_GROUP_SIZE", "MX_BLOCK"):
        assert getattr(arrms, name) == c[name], name


def test_status_strings():
    for s in (0, -1, -2, -3, -4):
        assert arrms.arrms_status_string(s) and arrms.arrms_status_string(s) != "unknown status"
    assert arrms.arrms_status_string(7) == "unknown status"


def _call(R=4, M=8, H=64, flags=0, eps=1e-6, entry=None, **over):
    ptr = {f"in{r}": BASE + (r if r < 8 else 16) * STRIDE for r in range(9)}
    ptr.update(residual=BASE + 10 * STRIDE, weight=BASE + 11 * STRIDE, out=BASE + 12 * STRIDE,
               residual_out=BASE + 13 * STRIDE, fp8_out=BASE + 14 * STRIDE,
               fp8_scale=BASE + 15 * STRIDE)
    ptr.update(over)
    rank_in = [ptr[f"in{r}"] for r in range(R)]
    fn = entry or arrms.arrms_fused_raw
    return fn(rank_in, R, ptr["residual"], ptr["weight"], ptr["out"], ptr["residual_out"], ptr["fp8_out"],
              ptr["fp8_scale"], M, H, eps, flags, None)


def test_zero_rows_is_ok_and_launches_nothing():
    assert _call(M=0) == arrms.OK
    assert _call(M=0, entry=arrms.arrms_fused_noalloc_raw) == arrms.OK
    assert arrms.arrms_query_path(0, 6144, 4, 0) == arrms.PATH_NONE


@pytest.mark.parametrize("kw", [
    dict(R=0), dict(R=9), dict(M=-1), dict(H=0), dict(flags=3), dict(flags=1 << 7), dict(eps=-1.0),
    dict(flags=arrms.FORCE_ONE_STAGE | arrms.FORCE_TWO_STAGE), dict(residual=None), dict(in2=None),
    dict(flags=arrms.FP8, fp8_scale=None), dict(H=60), dict(H=arrms.MAX_HIDDEN + 8),
    dict(flags=arrms.DTYPE_FP32 | arrms.FP8), dict(in1=BASE + STRIDE + 8), dict(out=BASE + STRIDE + 16),
])
def test_noalloc_checks_arguments_like_arrms_fused(kw):
    # the no-alloc form runs arrms_fused's argument checks before any device call
    want = _call(**kw)
    assert want != arrms.OK
    assert _call(entry=arrms.arrms_fused_noalloc_raw, **kw) == want


@pytest.mark.parametrize("kw", [
    dict(R=0), dict(R=9), dict(M=-1), dict(H=0), dict(flags=3), dict(flags=1 << 7),
    dict(flags=arrms.FORCE_ONE_STAGE | arrms.FORCE_TWO_STAGE), dict(eps=-1.0),
    dict(eps=float("nan")), dict(eps=float("inf")), dict(residual=None), dict(weight=None),
    dict(residual_out=None), dict(out=None), dict(in2=None),
    dict(flags=arrms.FP8, fp8_out=None), dict(flags=arrms.FP8, fp8_scale=None),
])
def test_invalid_arguments(kw):
    assert _call(**kw) == arrms.ERR_INVALID


@pytest.mark.parametrize("kw", [
    dict(H=60),                                  # 120 bytes per bf16 row: not 16-byte packs
    dict(H=6, flags=arrms.DTYPE_FP32),           # 24 bytes per fp32 row
    dict(H=arrms.MAX_HIDDEN + 8),
    dict(H=arrms.MAX_HIDDEN + 4, flags=arrms.DTYPE_FP32),  # fp32 row past the hidden cap
    dict(flags=arrms.DTYPE_FP32 | arrms.FP8),
    dict(in1=BASE + STRIDE + 8),                 # misaligned rank input
    dict(residual=BASE + 10 * STRIDE + 2),
    dict(out=BASE + 12 * STRIDE + 4),
    dict(flags=arrms.FP8, fp8_scale=BASE + 15 * STRIDE + 2),
])
def test_unsupported_layouts(kw):
    assert _call(**kw) == arrms.ERR_UNSUPPORTED


def test_overlap_rules():
    M, H = 8, 64
    nbytes = M * H * 2
    # out overlapping a rank input
    assert _call(out=BASE + STRIDE + 16) == arrms.ERR_INVALID
    # residual_out overlapping residual but not equal
    assert _call(residual_out=BASE + 10 * STRIDE + 16) == arrms.ERR_INVALID
    # out and residual_out overlapping each other
    assert _call(out=BASE + 13 * STRIDE + nbytes - 16) == arrms.ERR_INVALID
    # out overlapping the weight
    assert _call(out=BASE + 11 * STRIDE) == arrms.ERR_INVALID
    # fp8 scale inside the fp8 codes
    assert _call(flags=arrms.FP8, fp8_scale=BASE + 14 * STRIDE + 64) == arrms.ERR_INVALID
    # adjacent but not overlapping buffers are fine (validation passes; M = 0 stops before launch)
    assert _call(M=0, out=BASE + 13 * STRIDE + nbytes) == arrms.OK
    # repeated rank pointers are inputs only: allowed
    assert _call(M=0, in1=BASE) == arrms.OK


def test_query_path():
    for flags in (0, arrms.DTYPE_FP16, arrms.DTYPE_FP16 | arrms.GEMMA | arrms.FP8):
        assert arrms.arrms_query_path(1024, 6144, 4, flags) in (arrms.PATH_ONE_STAGE,
                                                                arrms.PATH_TWO_STAGE)
    assert arrms.arrms_query_path(1024, 6144, 4, arrms.FORCE_TWO_STAGE) == arrms.PATH_TWO_STAGE
    assert arrms.arrms_query_path(1024, 6144, 4, arrms.FORCE_ONE_STAGE) == arrms.PATH_ONE_STAGE
    assert arrms.arrms_query_path(1024, 60, 4, 0) == arrms.ERR_UNSUPPORTED
    assert arrms.arrms_query_path(1024, 64, 9, 0) == arrms.ERR_INVALID
    assert arrms.arrms_query_path(16, 512, 4, arrms.DTYPE_FP32 | arrms.FP8) == arrms.ERR_UNSUPPORTED
    # every dtype up to the hidden cap (fp32: 64 KiB rows)
    assert arrms.arrms_query_path(16, 16384, 4, 0) == arrms.PATH_ONE_STAGE
    assert arrms.arrms_query_path(16, 8196, 4, arrms.DTYPE_FP32) == arrms.PATH_ONE_STAGE
    assert arrms.arrms_query_path(16, 16384, 8, arrms.DTYPE_FP32) == arrms.PATH_ONE_STAGE
    assert arrms.arrms_query_path(16, 16388, 4, arrms.DTYPE_FP32) == arrms.ERR_UNSUPPORTED


def _call_strided(R=4, M=8, H=64, flags=0, eps=1e-6, ld=(64, 64, 64, 64, 64), **over):
    ptr = {f"in{r}": BASE + r * STRIDE for r in range(8)}
    ptr.update(residual=BASE + 10 * STRIDE, weight=BASE + 11 * STRIDE, out=BASE + 12 * STRIDE,
               residual_out=BASE + 13 * STRIDE, fp8_out=BASE + 14 * STRIDE,
               fp8_scale=BASE + 15 * STRIDE)
    ptr.update(over)
    rank_in = [ptr[f"in{r}"] for r in range(R)]
    return arrms.arrms_fused_strided_raw(rank_in, R, ptr["residual"], ptr["weight"], ptr["out"],
                                         ptr["residual_out"], ptr["fp8_out"], ptr["fp8_scale"], M, H,
                                         *ld, eps, flags, None)


def test_strided_argument_checks():
    assert _call_strided(M=0) == arrms.OK
    assert _call_strided(M=0, ld=(72, 80, 64, 96, 64)) == arrms.OK
    # a stride below the row is invalid, one that breaks 16-byte rows unsupported
    for i in range(4):
        ld = [64] * 5
        ld[i] = 56
        assert _call_strided(ld=tuple(ld)) == arrms.ERR_INVALID
        ld[i] = 68                                 # 136-byte bf16 rows
        assert _call_strided(ld=tuple(ld)) == arrms.ERR_UNSUPPORTED
    # fp8 stride counts bytes: >= H and a multiple of 8
    assert _call_strided(flags=arrms.FP8, ld=(64, 64, 64, 64, 48)) == arrms.ERR_INVALID
    assert _call_strided(flags=arrms.FP8, ld=(64, 64, 64, 64, 68)) == arrms.ERR_UNSUPPORTED
    assert _call_strided(M=0, flags=arrms.FP8, ld=(64, 64, 64, 64, 72)) == arrms.OK
    # FP8 with 8-byte code rows (H = 8) at unit stride
    assert _call_strided(M=0, H=8, flags=arrms.FP8, ld=(8, 8, 8, 8, 8)) == arrms.OK
    assert _call(M=0, H=8, flags=arrms.FP8) == arrms.OK
    # without FP8 the fp8 stride is ignored
    assert _call_strided(M=0, ld=(64, 64, 64, 64, 0)) == arrms.OK
    # fp32 rows: 4-element multiples
    assert _call_strided(flags=arrms.DTYPE_FP32, ld=(66, 64, 64, 64, 64)) == arrms.ERR_UNSUPPORTED
    assert _call_strided(M=0, flags=arrms.DTYPE_FP32, ld=(68, 64, 64, 64, 64)) == arrms.OK
    # in place needs equal residual strides
    assert _call_strided(residual_out=BASE + 10 * STRIDE, ld=(64, 64, 64, 80, 64)) == arrms.ERR_INVALID
    assert _call_strided(M=0, residual_out=BASE + 10 * STRIDE, ld=(64, 80, 64, 80, 64)) == arrms.OK


def test_strided_overlap_counts_the_padding():
    M, H, ld = 8, 64, 128
    span = ((M - 1) * ld + H) * 2
    lds = (ld, ld, ld, ld, ld)
    # out placed inside the padded span of residual_out overlaps it
    assert _call_strided(ld=lds, out=BASE + 13 * STRIDE + span - 16) == arrms.ERR_INVALID
    # ... and just past the span it does not (M = 0 stops before any launch)
    assert _call_strided(M=0, ld=lds, out=BASE + 13 * STRIDE + span) == arrms.OK


def _sum(R=4, n=4096, flags=0, out=BASE + 12 * STRIDE, **over):
    ptr = {f"in{r}": BASE + r * STRIDE for r in range(9)}
    ptr.update(over)
    return arrms.arrms_allreduce_sum_raw([ptr[f"in{r}"] for r in range(R)], R, out, n, flags, None)


def test_allreduce_sum_argument_checks():
    assert _sum(n=0) == arrms.OK
    assert _sum(n=0, out=BASE) == arrms.OK                   # in place on rank 0
    for kw in (dict(R=0), dict(R=9), dict(n=-8), dict(flags=3), dict(flags=arrms.GEMMA),
               dict(flags=arrms.FP8), dict(flags=arrms.FORCE_TWO_STAGE), dict(out=None),
               dict(in1=None), dict(out=BASE + STRIDE + 16)):
        assert _sum(**kw) == arrms.ERR_INVALID, kw
    for kw in (dict(n=4100), dict(n=2050, flags=arrms.DTYPE_FP32), dict(out=BASE + 12 * STRIDE + 8),
               dict(in3=BASE + 3 * STRIDE + 4)):
        assert _sum(**kw) == arrms.ERR_UNSUPPORTED, kw


def test_fused_config_argument_checks():
    ptr = [BASE + r * STRIDE for r in range(4)]
    args = (ptr, 4, BASE + 10 * STRIDE, BASE + 11 * STRIDE, BASE + 12 * STRIDE, BASE + 13 * STRIDE,
            None, None, 0, 64, 1e-6, 0)
    assert arrms.arrms_fused_config_raw(*args, 0, 0, 0, 0, None) == arrms.OK
    assert arrms.arrms_fused_config_raw(*args, 0, 0, 0, 0, None, load_window=2) == arrms.OK
    assert arrms.arrms_fused_config_raw(*args, 0, 0, 0, 0, None, load_window=3) == arrms.OK
    for bad in ((-1, 0, 0, 0, 0), (0, -64, 0, 0, 0), (0, 0, -1, 0, 0), (0, 0, 0, -5, 0), (0, 0, 0, 0, 4),
                (0, 0, 0, 0, -1)):
        ppt, tpr, rpb, blocks, win = bad
        assert arrms.arrms_fused_config_raw(*args, ppt, tpr, rpb, blocks, None, load_window=win) == \
            arrms.ERR_INVALID, bad


def _quant(R=4, M=8, H=256, flags=0, quant=2, eps=1e-6, **over):
    ptr = {f"in{r}": BASE + r * STRIDE for r in range(8)}
    ptr.update(residual=BASE + 10 * STRIDE, weight=BASE + 11 * STRIDE, out=None,
               residual_out=BASE + 13 * STRIDE, q_out=BASE + 14 * STRIDE, q_scale=BASE + 15 * STRIDE)
    ptr.update(over)
    return arrms.arrms_fused_quant_raw([ptr[f"in{r}"] for r in range(R)], R, ptr["residual"], ptr["weight"],
                                       ptr["out"], ptr["residual_out"], ptr["q_out"], ptr["q_scale"], M, H,
                                       eps, flags, quant, None)


def test_fused_quant_argument_checks():
    for q in (1, 2, 3):
        assert _quant(M=0, quant=q) == arrms.OK
        assert _quant(M=0, quant=q, flags=arrms.DTYPE_FP16 | arrms.GEMMA) == arrms.OK
    for kw in (dict(quant=0), dict(quant=4), dict(flags=arrms.FP8), dict(q_out=None), dict(q_scale=None),
               dict(residual_out=None)):
        assert _quant(**kw) == arrms.ERR_INVALID, kw
    # group sizes: per-group FP8 needs H % 128, MXFP4 H % 32; fp32 has no quant forms
    assert _quant(H=192, quant=2) == arrms.ERR_UNSUPPORTED
    assert _quant(M=0, H=192, quant=3) == arrms.OK
    assert _quant(H=80, quant=3) == arrms.ERR_UNSUPPORTED
    assert _quant(quant=2, flags=arrms.DTYPE_FP32) == arrms.ERR_UNSUPPORTED
    # MXFP4 scales are bytes: any alignment; FP8 group scales are fp32: 4-byte aligned
    assert _quant(M=0, quant=3, q_scale=BASE + 15 * STRIDE + 1) == arrms.OK
    assert _quant(quant=2, q_scale=BASE + 15 * STRIDE + 2) == arrms.ERR_UNSUPPORTED
    # overlap: the group scales [M][H/128] fp32 run into the codes
    M, H = 8, 256
    assert _quant(quant=2, q_scale=BASE + 14 * STRIDE + M * H - 4) == arrms.ERR_INVALID
    assert _quant(M=0, quant=2, q_scale=BASE + 14 * STRIDE + M * H) == arrms.OK
    # MXFP4 codes are [M][H/2]: scales right after them do not overlap
    assert _quant(M=0, quant=3, q_scale=BASE + 14 * STRIDE + M * H // 2) == arrms.OK
