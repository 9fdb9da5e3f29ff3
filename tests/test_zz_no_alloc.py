"""arrms_fused_noalloc on a GPU, through the C ABI: the same bits as arrms_fused
on both paths, two calls in a row (the second smaller, so it runs over what the
first left in the shared fixed staging region), no staging buffer reserved by
it, and a graph captured with no staging reserved replays correctly.
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

ONE, TWO = 16, 32


def _bufs(wl, mirror=True):
    dev = torch.device("cuda")
    T = gu.TORCH_T[wl.dtype]
    M, H = wl.M, wl.H
    fp8 = bool(wl.flags & 8)
    return {"out": gu.poison_(torch.empty(M, H, dtype=T, device=dev)) if (mirror or not fp8) else None,
            "residual_out": gu.poison_(torch.empty(M, H, dtype=T, device=dev)),
            "fp8": gu.poison_(torch.empty(M, H, dtype=torch.uint8, device=dev)) if fp8 else None,
            "scale": gu.poison_(torch.empty(M, dtype=torch.float32, device=dev)) if fp8 else None}


def _host(b):
    return {k: None if v is None else gu.host_bits(v) for k, v in b.items()}


def _run(fn, wl, xd, rd, wd, flags, mirror=True):
    b = _bufs(wl, mirror)
    fn(xd, rd, wd, b["out"], b["residual_out"], b["fp8"], b["scale"], eps=wl.eps, flags=flags, M=wl.M, H=wl.H)
    torch.cuda.synchronize()
    return _host(b)


def _same(a, b, label):
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], b[k]), f"{label}: {k}"


# the first call spans two chunks of the 16 MiB region (1365 rows of 6144 bf16
# fit), the second is smaller and of another type and epilogue
CASES = [wlmod.Workload("noalloc_big", R=4, M=2000, H=6144, row_scale=(0.1, 10.0)),
         wlmod.Workload("noalloc_small", R=3, M=300, H=2880, dtype="fp16", gemma=True, fp8=True, w_mean=0.0)]


def test_two_calls_in_a_row_match_arrms_fused():
    arrms.arrms_release_staging()
    assert arrms.arrms_staging_bytes() == 0
    dev = torch.device("cuda")
    got = []
    inputs = []
    for i, wl in enumerate(CASES):
        print(f"noalloc call {i}: {wl.name} R={wl.R} M={wl.M} H={wl.H} {wl.dtype} flags={wl.flags}", flush=True)
        xs, res, w = wlmod.make_inputs(wl, seed=20 + i)
        xd = [x.to(dev) for x in xs]
        rd, wd = res.to(dev), w.to(dev)
        inputs.append((xd, rd, wd))
        got.append({p: _run(arrms.arrms_fused_noalloc, wl, xd, rd, wd, wl.flags | f) for p, f in
                    (("two", TWO), ("one", ONE), ("auto", 0))})
        # the no-alloc path reserved nothing
        assert arrms.arrms_staging_bytes() == 0
    for i, wl in enumerate(CASES):
        xd, rd, wd = inputs[i]
        want = _run(arrms.arrms_fused, wl, xd, rd, wd, wl.flags | TWO)
        for p in ("two", "one", "auto"):
            _same(got[i][p], want, f"{wl.name}/{p}")
        # and the oracle agrees (the acceptance bars)
        xs, res, w = wlmod.make_inputs(wl, seed=20 + i)
        gu.compare(got[i]["two"], gu.run_oracle(wl, xs, res, w), wl.dtype, label=f"{wl.name}/oracle")


def test_capture_without_reserved_staging():
    wl = CASES[1].with_(M=700)
    dev = torch.device("cuda")
    xs, res, w = wlmod.make_inputs(wl, seed=31)
    xd = [x.to(dev) for x in xs]
    rd, wd = res.to(dev), w.to(dev)
    want = _run(arrms.arrms_fused, wl, xd, rd, wd, wl.flags | ONE)
    # the region's address is looked up on the first call on a device: outside capture
    _same(_run(arrms.arrms_fused_noalloc, wl, xd, rd, wd, wl.flags | ONE), want, "eager")
    arrms.arrms_release_staging()
    b = _bufs(wl)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        # arrms_fused cannot take the two-stage path here (nothing reserved) ...
        rc = arrms.arrms_fused_raw(xd, wl.R, rd, wd, b["out"], b["residual_out"], b["fp8"], b["scale"], wl.M, wl.H,
                                   wl.eps, wl.flags | TWO, s.cuda_stream)
        assert rc == arrms.ERR_NO_STAGING
        # ... the no-alloc form can
        arrms.arrms_fused_noalloc(xd, rd, wd, b["out"], b["residual_out"], b["fp8"], b["scale"], eps=wl.eps,
                                  flags=wl.flags | TWO, stream=s)
    torch.cuda.synchronize()
    assert arrms.arrms_staging_bytes() == 0
    other = CASES[0]
    oxs, ores, ow = wlmod.make_inputs(other, seed=32)
    oxd = [x.to(dev) for x in oxs]
    ord_, owd = ores.to(dev), ow.to(dev)
    for rep in range(3):
        for v in b.values():
            if v is not None:
                gu.poison_(v)
        g.replay()
        torch.cuda.synchronize()
        _same(_host(b), want, f"replay {rep}")
        # eager no-alloc work between replays overwrites the shared region
        _run(arrms.arrms_fused_noalloc, other, oxd, ord_, owd, other.flags | TWO)
    del g
