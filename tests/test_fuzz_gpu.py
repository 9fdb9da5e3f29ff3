"""Seeded random cases against the oracle, on a GPU: random rank counts, row
counts, hidden sizes (any multiple of one 16-byte pack), dtypes, gemma, every
output form (T, per-token FP8 with and without the mirror, per-group FP8,
MXFP4), both paths, and for the T and per-token forms random row padding
through arrms_fused_strided. Inputs follow the workloads' recipe with random
scales, so rows of very different magnitudes meet. Each case prints its
parameters before it runs; the bars are those of the other parity tests.
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

PATHS = {"one": 16, "two": 32}
N_CASES = 96


def _draw(i):
    rng = np.random.default_rng(1000 + i)
    dtype = ["bf16", "fp16", "fp32"][rng.integers(0, 3)]
    e = 4 if dtype == "fp32" else 2
    quant = 0 if dtype == "fp32" else int(rng.choice([0, 1, 1, 2, 3]))
    step = {0: 16 // e, 1: 16 // e, 2: 128, 3: 32}[quant]
    H = int(step * rng.integers(1, max(2, 4096 // step) + 1))
    M = int(rng.choice([1, 2, 3, 7, 16, 33, 64, 100, 257, 513, 1000]))
    R = int(rng.integers(1, 9))
    # fp16 keeps every sum finite (|x| well below 65504 / R)
    sigmas, top = ([0.01, 1.0, 4.0], 10.0) if dtype == "fp16" else ([0.01, 1.0, 30.0], 100.0)
    wl = wlmod.Workload(f"fuzz{i}", R=R, M=M, H=H, dtype=dtype, gemma=bool(rng.integers(0, 2)),
                        fp8=quant == 1, mirror=bool(rng.integers(0, 2)) if quant else True,
                        x_sigma=float(rng.choice(sigmas)),
                        row_scale=(0.01, top) if rng.integers(0, 2) else None,
                        w_mean=float(rng.choice([0.0, 1.0])), eps=float(rng.choice([1e-6, 1e-5, 0.0])))
    pad = int(rng.choice([0, 0, 8, 24])) * (16 // e)
    path = ["one", "two"][rng.integers(0, 2)]
    return wl, quant, pad, path, int(rng.integers(0, 1 << 30))


def _quant_flag(quant):
    return {0: 0, 1: oracle.FP8, 2: oracle.FP8_GROUP, 3: oracle.MXFP4}[quant]


@pytest.mark.parametrize("i", range(N_CASES))
def test_fuzz_case(i):
    wl, quant, pad, path, seed = _draw(i)
    print(f"fuzz case {i}: R={wl.R} M={wl.M} H={wl.H} {wl.dtype} gemma={wl.gemma} quant={quant} "
          f"mirror={wl.mirror} pad={pad} path={path} eps={wl.eps} seed={seed}", flush=True)
    xs, res, w = wlmod.make_inputs(wl, seed=seed)
    dt = wlmod.DT_CODE[wl.dtype]
    want = oracle.fused([gu.host_bits(x) for x in xs], gu.host_bits(res), gu.host_bits(w), wl.eps,
                        dt | (oracle.GEMMA if wl.gemma else 0) | _quant_flag(quant), want_out=wl.mirror)
    dev = torch.device("cuda")
    T = gu.TORCH_T[wl.dtype]
    M, H = wl.M, wl.H
    flags = dt | (arrms.GEMMA if wl.gemma else 0) | PATHS[path]
    arrms.arrms_reserve_staging(0)
    if quant in (0, 1):
        # arrms_fused_strided: every matrix a window of a wider, poisoned allocation
        def win(src=None, dtype=T):
            base = gu.poison_(torch.empty(M, H + pad, dtype=dtype, device=dev))
            v = base[:, :H]
            if src is not None:
                v.copy_(src)
            return v
        xd = [win(x) for x in xs]
        rd = win(res)
        out = win() if wl.mirror else None
        rout = win()
        q = win(dtype=torch.uint8) if quant == 1 else None
        sc = gu.poison_(torch.empty(M, dtype=torch.float32, device=dev)) if quant == 1 else None
        arrms.arrms_fused_strided(xd, rd, w.to(dev), out, rout, q, sc, eps=wl.eps,
                                  flags=flags | (arrms.FP8 if quant == 1 else 0))
    else:
        qshape = (M, H // 2) if quant == 3 else (M, H)
        sshape, sdt = ((M, H // 32), torch.uint8) if quant == 3 else ((M, H // 128), torch.float32)
        xd = [x.to(dev) for x in xs]
        rd = res.to(dev)
        out = gu.poison_(torch.empty(M, H, dtype=T, device=dev)) if wl.mirror else None
        rout = gu.poison_(torch.empty(M, H, dtype=T, device=dev))
        q = gu.poison_(torch.empty(qshape, dtype=torch.uint8, device=dev))
        sc = gu.poison_(torch.empty(sshape, dtype=sdt, device=dev))
        arrms.arrms_fused_quant(xd, rd, w.to(dev), out, rout, q, sc, eps=wl.eps, flags=flags, quant=quant)
    torch.cuda.synchronize()
    got = {"out": None if out is None else gu.host_bits(out), "residual_out": gu.host_bits(rout),
           "fp8": None if q is None else gu.host_bits(q), "scale": None if sc is None else gu.host_bits(sc)}
    label = f"fuzz{i}"
    if quant in (0, 1):
        gu.compare(got, want, wl.dtype, label=label)
    else:
        assert np.array_equal(got["residual_out"], want["residual_out"]), f"{label}: residual_out"
        if want["out"] is not None:
            assert np.array_equal(got["out"], want["out"]), f"{label}: out"
        assert np.array_equal(got["fp8"], want["fp8"]), f"{label}: codes"
        assert np.array_equal(got["scale"].view(np.uint8), want["scale"].view(np.uint8)), f"{label}: scales"
