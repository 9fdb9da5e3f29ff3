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
