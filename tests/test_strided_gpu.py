"""Parity of arrms_fused_strided (row-padded matrices) with the oracle, on a GPU.

Every tensor lives inside a wider, NaN-poisoned allocation: the rows of the
operation are a column window of it, at a per-tensor row stride. The results
in the window must equal the oracle's on the compact copies of the same
inputs (bit for bit, as for arrms_fused), and every byte outside the window
must still hold the poison afterwards. Both paths run every case.
"""
import numpy as np
import pytest
import torch

from all_reduce_residual_rank_amd import workloads as wlmod
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from all_reduce_residual_rank_amd import arrms
else:  # pragma: no cover - collected on CPU only with -m gpu deselected
    arrms = None

PATHS = {"one": 16, "two": 32}


def _padded(M, ld, col, H, dtype, fill=None):
    """A poisoned [M][ld] allocation and its [M][H] window starting at column col."""
    dev = torch.device("cuda")
    base = gu.poison_(torch.empty(M, ld, dtype=dtype, device=dev))
    win = base[:, col:col + H]
    if fill is not None:
        win.copy_(fill)
    return base, win


def _outside(base: torch.Tensor, col: int, H: int) -> np.ndarray:
    b = gu.host_bits(base)
    mask = np.ones(b.shape, dtype=bool)
    mask[:, col:col + H] = False
    return b[mask].view(np.uint8)


def _run_strided(wl, xs, res, w, path, pads, inplace=False):
    """pads: dict tensor-name -> (extra columns, column offset); fp8 in bytes."""
    T = gu.TORCH_T[wl.dtype]
    M, H = wl.M, wl.H
    flags = wl.flags | PATHS[path]
    fp8 = bool(flags & arrms.FP8)
    keep = {}

    def mk(name, dtype, fill=None):
        extra, col = pads.get(name, (0, 0))
        base, win = _padded(M, H + extra, col, H, dtype, fill)
        keep[name] = (base, col, win)
        return win

    xin = [mk(f"in{r}", T, xs[r].cuda()) if r == 0 else None for r in range(wl.R)]
    # all rank inputs share one stride: same padding as rank 0
    for r in range(1, wl.R):
        extra, col = pads.get("in0", (0, 0))
        base, win = _padded(M, H + extra, col, H, T, xs[r].cuda())
        keep[f"in{r}"] = (base, col, win)
        xin[r] = win
    rd = mk("res", T, res.cuda())
    wd = w.cuda()
    out = mk("out", T) if (wl.mirror or not fp8) else None
    rout = rd if inplace else mk("rout", T)
    q = mk("q", torch.uint8) if fp8 else None
    sc = gu.poison_(torch.empty(M, dtype=torch.float32, device="cuda")) if fp8 else None
    print(f"strided case {wl.name} R={wl.R} M={M} H={H} {wl.dtype} flags={flags} pads={pads} "
          f"inplace={inplace}", flush=True)
    arrms.arrms_fused_strided(xin, rd, wd, out, rout, q, sc, eps=wl.eps, flags=flags)
    torch.cuda.synchronize()
    got = {"out": None if out is None else gu.host_bits(out),
           "residual_out": gu.host_bits(rout), "fp8": None if q is None else gu.host_bits(q),
           "scale": None if sc is None else gu.host_bits(sc)}
    for name, (base, col, _) in keep.items():
        assert np.all(_outside(base, col, H) == 0xFF), f"{name}: padding written"
    # the inputs themselves must be unchanged (except the residual in place)
    for r in range(wl.R):
        assert np.array_equal(gu.host_bits(keep[f"in{r}"][2]), gu.host_bits(xs[r]))
    return got


PADS = {
    "all8": {"in0": (8, 0), "res": (8, 0), "out": (8, 0), "rout": (8, 0), "q": (16, 0)},
    "mixed": {"in0": (64, 8), "res": (24, 16), "out": (8, 8), "rout": (136, 0), "q": (48, 32)},
    "in_only": {"in0": (512, 256)},
    "out_only": {"out": (16, 0), "rout": (8, 8), "q": (16, 16)},
}


@pytest.mark.parametrize("path", ["one", "two"])
@pytest.mark.parametrize("pad", list(PADS), ids=str)
@pytest.mark.parametrize("wl", [
    wlmod.Workload("s_bf16", R=4, M=121, H=2880, row_scale=(0.1, 10.0)),
    wlmod.Workload("s_fp16_fp8", R=4, M=64, H=6144, dtype="fp16", gemma=True, fp8=True, mirror=True,
                   x_sigma=2.0, w_mean=0.0),
    wlmod.Workload("s_bf16_fp8_nomirror", R=2, M=33, H=512, fp8=True, mirror=False),
    wlmod.Workload("s_fp32", R=8, M=65, H=512, dtype="fp32"),
    wlmod.Workload("s_bf16_r8_wide", R=8, M=17, H=7168, eps=1e-5),
], ids=lambda w: w.name)
def test_strided_matches_oracle(wl, pad, path):
    pads = dict(PADS[pad])
    if wl.dtype == "fp32":
        # fp32 rows: column offsets and padding in multiples of 4 elements
        pads = {k: (e // 2 if k != "q" else e, c // 2 if k != "q" else c) for k, (e, c) in pads.items()}
    xs, res, w = wlmod.make_inputs(wl, seed=5)
    want = gu.run_oracle(wl, xs, res, w)
    got = _run_strided(wl, xs, res, w, path, pads)
    gu.compare(got, want, wl.dtype, label=f"{wl.name}/{pad}/{path}")


@pytest.mark.parametrize("path", ["one", "two"])
def test_strided_in_place_residual(path):
    wl = wlmod.Workload("s_inplace", R=4, M=100, H=2880, dtype="fp16")
    xs, res, w = wlmod.make_inputs(wl, seed=6)
    want = gu.run_oracle(wl, xs, res, w)
    got = _run_strided(wl, xs, res, w, path, {"in0": (32, 16), "res": (40, 8), "out": (8, 0)},
                       inplace=True)
    gu.compare(got, want, wl.dtype, label=f"inplace/{path}")


def test_unit_strides_equal_arrms_fused():
    wl = wlmod.Workload("s_unit", R=4, M=50, H=2880, fp8=True, mirror=True)
    xs, res, w = wlmod.make_inputs(wl, seed=8)
    a = gu.run_hip(wl, xs, res, w)
    b = _run_strided(wl, xs, res, w, "one", {})
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k]), k


def test_small_staging_chunks_with_strides():
    # the two-stage chunk loop with strided inputs reduces row by row
    torch.cuda.synchronize()
    arrms.arrms_release_staging()
    arrms.arrms_reserve_staging(5 * 2880 * 2 + 16)
    try:
        wl = wlmod.Workload("s_chunks", R=3, M=23, H=2880, fp8=True, mirror=True)
        xs, res, w = wlmod.make_inputs(wl, seed=9)
        want = gu.run_oracle(wl, xs, res, w)
        got = _run_strided(wl, xs, res, w, "two", PADS["mixed"])
        gu.compare(got, want, wl.dtype, label="chunks")
    finally:
        torch.cuda.synchronize()
        arrms.arrms_release_staging()


@pytest.mark.parametrize("path", ["one", "two"])
def test_fp8_rows_eight_byte_aligned(path):
    # FP8 code rows at a stride of 8 mod 16 bytes, and 8-byte code rows (H = 8)
    for wl, pads in ((wlmod.Workload("s_q8", R=2, M=31, H=512, fp8=True, mirror=True),
                      {"q": (8, 0), "in0": (8, 0)}),
                     (wlmod.Workload("s_h8", R=3, M=19, H=8, fp8=True, mirror=True),
                      {"q": (8, 0), "res": (8, 8), "out": (16, 0)})):
        xs, res, w = wlmod.make_inputs(wl, seed=11)
        want = gu.run_oracle(wl, xs, res, w)
        got = _run_strided(wl, xs, res, w, path, pads)
        gu.compare(got, want, wl.dtype, label=f"{wl.name}/{path}")


def test_strided_graph_replay():
    # arrms_fused_strided captured once per path and replayed with new inputs
    wl = wlmod.Workload("s_graph", R=4, M=90, H=2880, row_scale=(0.1, 10.0))
    arrms.arrms_reserve_staging(0)
    dev = torch.device("cuda")
    M, H = wl.M, wl.H
    xs0, res0, w0 = wlmod.make_inputs(wl, seed=0)
    xin = [_padded(M, H + 32, 16, H, torch.bfloat16, x.cuda())[1] for x in xs0]
    _, rd = _padded(M, H + 8, 0, H, torch.bfloat16, res0.cuda())
    wd = w0.to(dev)
    bufs, graphs = {}, {}
    for path in ("one", "two"):
        ob, out = _padded(M, H + 64, 8, H, torch.bfloat16)
        rb, rout = _padded(M, H + 8, 8, H, torch.bfloat16)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            arrms.arrms_fused_strided(xin, rd, wd, out, rout, eps=wl.eps, flags=wl.flags | PATHS[path],
                                      stream=s)
        torch.cuda.current_stream().wait_stream(s)
        bufs[path], graphs[path] = (ob, out, rb, rout), g
    for step in range(3):
        xs, res, w = wlmod.make_inputs(wl, seed=30 + step)
        for d, h in zip(xin, xs):
            d.copy_(h)
        rd.copy_(res)
        wd.copy_(w)
        want = gu.run_oracle(wl, xs, res, w)
        for path in ("one", "two"):
            ob, out, rb, rout = bufs[path]
            gu.poison_(ob)
            gu.poison_(rb)
            torch.cuda.synchronize()
            print(f"strided graph replay path={path} step={step}", flush=True)
            graphs[path].replay()
            torch.cuda.synchronize()
            got = {"out": gu.host_bits(out), "residual_out": gu.host_bits(rout), "fp8": None, "scale": None}
            gu.compare(got, want, "bf16", label=f"strided-graph-{path}-{step}")
            assert np.all(_outside(ob, 8, H) == 0xFF) and np.all(_outside(rb, 8, H) == 0xFF)
