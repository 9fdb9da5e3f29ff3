"""Non-finite inputs on a GPU, against the oracle's reading (IEEE arithmetic;
a maximum over |y| covering a NaN is NaN; one sign-free E4M3 NaN code 0x7F;
NaN elements of a NaN-scaled MXFP4 block coded 0x7): NaN and infinite
weights (one column of every row) and residual elements (one row), for the T
output and all three quant forms, on both paths.

NaN payloads and signs in the T outputs and the fp32 scales are not part of
the reading: those compare as "NaN at the same places, equal bits elsewhere".
Code and E8M0 scale bytes compare exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from all_reduce_residual_rank_amd import workloads as wlmod
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from all_reduce_residual_rank_amd import arrms
else:  # pragma: no cover - collected on CPU only with -m gpu deselected
    arrms = None

R, M, H = 3, 8, 512
PATHS = {"one": 16, "two": 32}
NAN = {"bf16": 0x7FC0, "fp16": 0x7E00}
INF = {"bf16": 0x7F80, "fp16": 0x7C00}
QFLAG = {0: 0, 1: oracle.FP8, 2: oracle.FP8_GROUP, 3: oracle.MXFP4}


def _case(dtype, kind):
    wl = wlmod.Workload("nonfinite", R=R, M=M, H=H, dtype=dtype)
    xs, res, w = wlmod.make_inputs(wl, seed=13)
    xs = [gu.host_bits(x) for x in xs]
    res, w = gu.host_bits(res), gu.host_bits(w)
    if kind == "nan_weight":
        w[37] = NAN[dtype]
    elif kind == "inf_weight":
        w[100] = INF[dtype]
    elif kind == "nan_residual":
        res[2, 300] = NAN[dtype]
    elif kind == "inf_residual":
        res[5, 10] = INF[dtype] | 0x8000
    return xs, res, w


def _to_dev(a, dtype):
    t = torch.from_numpy(a.view(np.int16).copy()).view(gu.TORCH_T[dtype])
    return t.to("cuda")


def _run_hip(xs, res, w, dtype, quant, path):
    dev = torch.device("cuda")
    T = gu.TORCH_T[dtype]
    xd = [_to_dev(x, dtype) for x in xs]
    rd, wd = _to_dev(res, dtype), _to_dev(w, dtype)
    out = gu.poison_(torch.empty(M, H, dtype=T, device=dev))
    rout = gu.poison_(torch.empty(M, H, dtype=T, device=dev))
    flags = wlmod.DT_CODE[dtype] | PATHS[path]
    q = sc = None
    print(f"nonfinite case {dtype} quant={quant} path={path}", flush=True)
    if quant == 0:
        arrms.arrms_fused(xd, rd, wd, out, rout, eps=1e-6, flags=flags)
    else:
        qshape = (M, H // 2) if quant == 3 else (M, H)
        q = gu.poison_(torch.empty(qshape, dtype=torch.uint8, device=dev))
        if quant == 1:
            sc = gu.poison_(torch.empty(M, dtype=torch.float32, device=dev))
        elif quant == 2:
            sc = gu.poison_(torch.empty(M, H // 128, dtype=torch.float32, device=dev))
        else:
            sc = gu.poison_(torch.empty(M, H // 32, dtype=torch.uint8, device=dev))
        arrms.arrms_fused_quant(xd, rd, wd, out, rout, q, sc, eps=1e-6, flags=flags, quant=quant)
    torch.cuda.synchronize()
    return {"out": gu.host_bits(out), "residual_out": gu.host_bits(rout),
            "fp8": None if q is None else gu.host_bits(q), "scale": None if sc is None else gu.host_bits(sc)}


def _same_t(got, want, dtype, label):
    inf = INF[dtype]
    gn, wn = (got & 0x7FFF) > inf, (want & 0x7FFF) > inf
    assert np.array_equal(gn, wn), f"{label}: NaN positions differ"
    assert np.array_equal(got[~wn], want[~wn]), f"{label}: {(got[~wn] != want[~wn]).sum()} values differ"


def _same_f32(got, want, label):
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), f"{label}: NaN scales differ"
    assert np.array_equal(got[~wn].view(np.uint32), want[~wn].view(np.uint32)), f"{label}: scales differ"


@pytest.mark.parametrize("path", ["one", "two"])
@pytest.mark.parametrize("quant", [0, 1, 2, 3], ids=["t", "fp8", "fp8group", "mxfp4"])
@pytest.mark.parametrize("kind", ["nan_weight", "inf_weight", "nan_residual", "inf_residual"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_nonfinite_matches_oracle(dtype, kind, quant, path):
    xs, res, w = _case(dtype, kind)
    want = oracle.fused(xs, res, w, 1e-6, wlmod.DT_CODE[dtype] | QFLAG[quant], want_out=True)
    got = _run_hip(xs, res, w, dtype, quant, path)
    label = f"{dtype}/{kind}/q{quant}/{path}"
    _same_t(got["residual_out"], want["residual_out"], dtype, label + " residual_out")
    _same_t(got["out"], want["out"], dtype, label + " out")
    if quant:
        assert np.array_equal(got["fp8"], want["fp8"]), \
            f"{label}: {(got['fp8'] != want['fp8']).sum()} code bytes differ"
        if quant == 3:
            assert np.array_equal(got["scale"], want["scale"]), f"{label}: E8M0 scales differ"
        else:
            _same_f32(got["scale"], want["scale"], label)
