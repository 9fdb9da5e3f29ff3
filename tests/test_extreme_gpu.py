"""Finite inputs at the ends of the exponent range, on a GPU, against the oracle.

bf16 shares fp32's exponent range, so the product h * w of a row element and
its weight can overflow fp32 (|h|, |w| near 2^100) or fall below its normal
range (|h|, |w| near 2^-100), while the normalised value h * w * rstd is an
ordinary number: the oracle forms that product in fp64 (one rounding of
(h * w_eff) * rstd to T), and the kernels must give the same bits. With
eps = 0 a row of tiny values has a huge rstd, so even a product that
underflows to zero in fp32 can normalise to a nonzero output. fp16 rows take
values across fp16's whole range (subnormals to 65504) with eps = 0.

Every output is compared bit for bit: residual_out, the T output, and with
per-token FP8 the codes and the fp32 scales.
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

R, M, H = 2, 6, 512
PATHS = {"one": 16, "two": 32}

# kind: (dtype, eps, h exponents (lo, hi) or a fixed scale, w exponents or a fixed scale)
KINDS = {
    # h ~ 2^100, w ~ 2^100: h * w ~ 2^200 is beyond fp32; y ~ 2^100
    "bf16_product_overflow": ("bf16", 1e-6, 100, 100),
    # h ~ 2^-100, w ~ 2^-40: h * w ~ 2^-140 is an fp32 subnormal (bits lost); y ~ 2^-40
    "bf16_product_subnormal": ("bf16", 0.0, -100, -40),
    # h ~ 2^-100, w ~ 2^-60: h * w ~ 2^-160 is zero in fp32; rstd ~ 2^100, y ~ 2^-60
    "bf16_product_zero": ("bf16", 0.0, -100, -60),
    # every element its own exponent: h in 2^[-100, 100], w in 2^[-60, 60]
    "bf16_wide_range": ("bf16", 1e-6, (-100, 100), (-60, 60)),
    "bf16_wide_range_eps0": ("bf16", 0.0, (-100, 100), (-60, 60)),
    # fp16 from subnormals to the top of the range
    "fp16_wide_range_eps0": ("fp16", 0.0, (-24, 11), (-14, 4)),
}


def _draw(shape, exps, g):
    v = torch.randn(shape, generator=g, dtype=torch.float64)
    v = torch.where(v.abs() < 0.25, torch.full_like(v, 0.5), v)  # keep every element near its exponent
    if isinstance(exps, tuple):
        e = torch.randint(exps[0], exps[1] + 1, shape, generator=g).to(torch.float64)
    else:
        e = torch.full(shape, float(exps), dtype=torch.float64)
    return v * torch.pow(2.0, e)


def _case(kind, seed=7):
    dtype, eps, hexp, wexp = KINDS[kind]
    T = gu.TORCH_T[dtype]
    g = torch.Generator().manual_seed(seed)
    xs = [_draw((M, H), hexp, g).to(T) for _ in range(R)]
    res = _draw((M, H), hexp, g).to(T)
    w = _draw((H,), wexp, g).abs().to(T)
    return dtype, eps, xs, res, w


def _run_hip(dtype, eps, xs, res, w, fp8, path):
    dev = torch.device("cuda")
    T = gu.TORCH_T[dtype]
    xd = [x.to(dev) for x in xs]
    rd, wd = res.to(dev), w.to(dev)
    out = gu.poison_(torch.empty(M, H, dtype=T, device=dev))
    rout = gu.poison_(torch.empty(M, H, dtype=T, device=dev))
    q = gu.poison_(torch.empty(M, H, dtype=torch.uint8, device=dev)) if fp8 else None
    sc = gu.poison_(torch.empty(M, dtype=torch.float32, device=dev)) if fp8 else None
    flags = wlmod.DT_CODE[dtype] | PATHS[path] | (arrms.FP8 if fp8 else 0)
    arrms.arrms_fused(xd, rd, wd, out, rout, q, sc, eps=eps, flags=flags)
    torch.cuda.synchronize()
    return {"out": gu.host_bits(out), "residual_out": gu.host_bits(rout),
            "fp8": None if q is None else gu.host_bits(q), "scale": None if sc is None else gu.host_bits(sc)}


@pytest.mark.parametrize("path", ["one", "two"])
@pytest.mark.parametrize("fp8", [False, True], ids=["t", "fp8"])
@pytest.mark.parametrize("kind", list(KINDS))
def test_extreme_exponents_match_oracle(kind, fp8, path):
    dtype, eps, xs, res, w = _case(kind)
    print(f"extreme case {kind} fp8={fp8} path={path}", flush=True)
    hb = [gu.host_bits(x) for x in xs]
    want = oracle.fused(hb, gu.host_bits(res), gu.host_bits(w), eps,
                        wlmod.DT_CODE[dtype] | (oracle.FP8 if fp8 else 0), want_out=True)
    yv = gu._values(want["out"], dtype)
    assert np.isfinite(yv).all() and (yv != 0).mean() > 0.5, "the case should normalise to ordinary values"
    got = _run_hip(dtype, eps, xs, res, w, fp8, path)
    label = f"{kind}/{'fp8' if fp8 else 't'}/{path}"
    assert np.array_equal(got["residual_out"], want["residual_out"]), f"{label}: residual_out differs"
    bad = got["out"] != want["out"]
    assert not bad.any(), f"{label}: {bad.sum()} outputs differ, e.g. got {got['out'][bad][:4]} want {want['out'][bad][:4]}"
    if fp8:
        assert np.array_equal(got["scale"].view(np.uint32), want["scale"].view(np.uint32)), f"{label}: scales differ"
        assert np.array_equal(got["fp8"], want["fp8"]), f"{label}: {(got['fp8'] != want['fp8']).sum()} codes differ"


# ---- all-zero rows with eps = 0: rstd = 1/sqrt(0) = inf and y = 0 * w * inf is
# NaN in every column (IEEE arithmetic, as the oracle reads it); the other
# rows are ordinary. Every output form, both paths; NaN payloads and signs are
# not part of the reading, so T values and fp32 scales compare as "NaN at the
# same places, equal bits elsewhere", codes and E8M0 scales exactly.
QFLAG = {0: 0, 1: oracle.FP8, 2: oracle.FP8_GROUP, 3: oracle.MXFP4}
INF = {"bf16": 0x7F80, "fp16": 0x7C00}


def _same_t(got, want, dtype, label):
    gn, wn = (got & 0x7FFF) > INF[dtype], (want & 0x7FFF) > INF[dtype]
    assert np.array_equal(gn, wn), f"{label}: NaN positions differ"
    assert np.array_equal(got[~wn], want[~wn]), f"{label}: {(got[~wn] != want[~wn]).sum()} values differ"


@pytest.mark.parametrize("path", ["one", "two"])
@pytest.mark.parametrize("quant", [0, 1, 2, 3], ids=["t", "fp8", "fp8group", "mxfp4"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_zero_rows_eps0_match_oracle(dtype, quant, path):
    T = gu.TORCH_T[dtype]
    g = torch.Generator().manual_seed(11)
    xs = [torch.randn(M, H, generator=g).to(T) for _ in range(R)]
    res = torch.randn(M, H, generator=g).to(T)
    w = (torch.randn(H, generator=g) * 0.1 + 1.0).to(T)
    for r in (1, 4):
        for x in xs:
            x[r] = 0
        res[r] = 0
    print(f"zero rows eps=0 {dtype} quant={quant} path={path}", flush=True)
    want = oracle.fused([gu.host_bits(x) for x in xs], gu.host_bits(res), gu.host_bits(w), 0.0,
                        wlmod.DT_CODE[dtype] | QFLAG[quant], want_out=True)
    dev = torch.device("cuda")
    xd = [x.to(dev) for x in xs]
    rd, wd = res.to(dev), w.to(dev)
    out = gu.poison_(torch.empty(M, H, dtype=T, device=dev))
    rout = gu.poison_(torch.empty(M, H, dtype=T, device=dev))
    flags = wlmod.DT_CODE[dtype] | PATHS[path]
    q = sc = None
    if quant == 0:
        arrms.arrms_fused(xd, rd, wd, out, rout, eps=0.0, flags=flags)
    else:
        q = gu.poison_(torch.empty((M, H // 2) if quant == 3 else (M, H), dtype=torch.uint8, device=dev))
        if quant == 1:
            sc = gu.poison_(torch.empty(M, dtype=torch.float32, device=dev))
        elif quant == 2:
            sc = gu.poison_(torch.empty(M, H // 128, dtype=torch.float32, device=dev))
        else:
            sc = gu.poison_(torch.empty(M, H // 32, dtype=torch.uint8, device=dev))
        arrms.arrms_fused_quant(xd, rd, wd, out, rout, q, sc, eps=0.0, flags=flags, quant=quant)
    torch.cuda.synchronize()
    label = f"zero rows {dtype}/q{quant}/{path}"
    assert np.array_equal(gu.host_bits(rout), want["residual_out"]), f"{label}: residual_out differs"
    got_out = gu.host_bits(out)
    assert ((want["out"][1] & 0x7FFF) > INF[dtype]).all(), "a zero row normalises to NaN with eps = 0"
    _same_t(got_out, want["out"], dtype, label + " out")
    if quant:
        assert np.array_equal(gu.host_bits(q), want["fp8"]), f"{label}: code bytes differ"
        gs, ws = gu.host_bits(sc), want["scale"]
        if quant == 3:
            assert np.array_equal(gs, ws), f"{label}: E8M0 scales differ"
        else:
            gn, wn = np.isnan(gs), np.isnan(ws)
            assert np.array_equal(gn, wn), f"{label}: NaN scales differ"
            assert np.array_equal(gs[~wn].view(np.uint32), ws[~wn].view(np.uint32)), f"{label}: scales differ"
