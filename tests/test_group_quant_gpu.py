"""Parity of the per-group FP8 and MXFP4 outputs (arrms_fused_quant) with the
oracle, on a GPU: codes, scales, the T mirror and residual_out, bit for bit,
on both paths. Outputs are poisoned before each call; code and scale buffers
are followed by poisoned guard bytes that must survive.
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
GUARD = 64


def _shapes(quant, M, H):
    if quant == 2:  # per-group FP8
        return (M, H), np.uint8, (M, H // 128), torch.float32
    return (M, H // 2), np.uint8, (M, H // 32), torch.uint8


def _run(wl, xs, res, w, quant, path, mirror):
    dev = torch.device("cuda")
    T = gu.TORCH_T[wl.dtype]
    M, H = wl.M, wl.H
    qshape, _, sshape, sdt = _shapes(quant, M, H)
    xd = [x.to(dev) for x in xs]
    rd, wd = res.to(dev), w.to(dev)
    out = gu.poison_(torch.empty(M, H, dtype=T, device=dev)) if mirror else None
    rout = gu.poison_(torch.empty(M, H, dtype=T, device=dev))
    qbuf = gu.poison_(torch.empty(qshape[0] * qshape[1] + GUARD, dtype=torch.uint8, device=dev))
    sbuf = gu.poison_(torch.empty(sshape[0] * sshape[1] * (4 if sdt == torch.float32 else 1) + GUARD,
                                  dtype=torch.uint8, device=dev))
    flags = wl.flags & ~oracle.FP8 | PATHS[path]
    print(f"group-quant case {wl.name} R={wl.R} M={M} H={H} {wl.dtype} quant={quant} path={path} "
          f"mirror={mirror}", flush=True)
    arrms.arrms_fused_quant(xd, rd, wd, out, rout, qbuf, sbuf, eps=wl.eps, flags=flags, quant=quant, M=M, H=H)
    torch.cuda.synchronize()
    qb = gu.host_bits(qbuf)
    sb = gu.host_bits(sbuf)
    nq = qshape[0] * qshape[1]
    ns = len(sb) - GUARD
    assert np.all(qb[nq:] == 0xFF) and np.all(sb[ns:] == 0xFF), "write past the end"
    scale = sb[:ns].view(np.float32).reshape(sshape) if sdt == torch.float32 else sb[:ns].reshape(sshape)
    return {"out": None if out is None else gu.host_bits(out), "residual_out": gu.host_bits(rout),
            "fp8": qb[:nq].reshape(qshape), "scale": scale}


def _oracle(wl, xs, res, w, quant, mirror):
    dt = wlmod.DT_CODE[wl.dtype]
    qf = oracle.FP8_GROUP if quant == 2 else oracle.MXFP4
    return oracle.fused([gu.host_bits(x) for x in xs], gu.host_bits(res), gu.host_bits(w), wl.eps,
                        dt | (oracle.GEMMA if wl.gemma else 0) | qf, want_out=mirror)


def _check(got, want, label):
    assert np.array_equal(got["residual_out"], want["residual_out"]), f"{label}: residual_out"
    if want["out"] is not None:
        assert np.array_equal(got["out"], want["out"]), f"{label}: out"
    d = got["fp8"] != want["fp8"]
    assert not d.any(), f"{label}: {d.sum()} code bytes differ"
    s = got["scale"].view(np.uint8) != want["scale"].view(np.uint8)
    assert not s.any(), f"{label}: {s.sum()} scale bytes differ"


WORKLOADS = [
    wlmod.Workload("q_bf16_6144", R=4, M=97, H=6144, row_scale=(0.1, 10.0)),
    wlmod.Workload("q_fp16_gemma_6144", R=4, M=64, H=6144, dtype="fp16", gemma=True, x_sigma=2.0,
                   w_mean=0.0),
    wlmod.Workload("q_bf16_r8_7168", R=8, M=33, H=7168, eps=1e-5),
    wlmod.Workload("q_fp16_r1_512", R=1, M=130, H=512, dtype="fp16"),
    wlmod.Workload("q_bf16_r3_128", R=3, M=17, H=128, gemma=True, w_mean=0.0),
]


@pytest.mark.parametrize("path", ["one", "two"])
@pytest.mark.parametrize("quant", [2, 3], ids=["fp8group", "mxfp4"])
@pytest.mark.parametrize("wl", WORKLOADS, ids=lambda w: w.name)
def test_group_quant_matches_oracle(wl, quant, path):
    xs, res, w = wlmod.make_inputs(wl, seed=21)
    for mirror in (True, False):
        want = _oracle(wl, xs, res, w, quant, mirror)
        got = _run(wl, xs, res, w, quant, path, mirror)
        _check(got, want, f"{wl.name}/q{quant}/{path}/mirror{mirror}")


# every R: with 2 to 6 ranks the group forms write residual_out after their
# codes, otherwise pack by pack (or after the reduction when the window throttles)
@pytest.mark.parametrize("path", ["one", "two"])
@pytest.mark.parametrize("quant", [2, 3], ids=["fp8group", "mxfp4"])
@pytest.mark.parametrize("R", range(1, 9))
def test_group_quant_every_rank_count(R, quant, path):
    wl = wlmod.Workload(f"q_rsweep_r{R}", R=R, M=200, H=6144, dtype="fp16", gemma=True, w_mean=0.0)
    xs, res, w = wlmod.make_inputs(wl, seed=60 + R)
    want = _oracle(wl, xs, res, w, quant, False)
    got = _run(wl, xs, res, w, quant, path, False)
    _check(got, want, f"{wl.name}/q{quant}/{path}")


@pytest.mark.parametrize("wl", [wlmod.Workload("mx_2880", R=4, M=121, H=2880),
                                wlmod.Workload("mx_fp16_96", R=2, M=40, H=96, dtype="fp16")],
                         ids=lambda w: w.name)
def test_mxfp4_ragged_rows(wl):
    # H a multiple of 32 but not of 128, rows that do not fill the last tile
    xs, res, w = wlmod.make_inputs(wl, seed=5)
    for path in ("one", "two"):
        _check(_run(wl, xs, res, w, 3, path, True), _oracle(wl, xs, res, w, 3, True), f"{wl.name}/{path}")


@pytest.mark.parametrize("quant", [2, 3], ids=["fp8group", "mxfp4"])
def test_group_quant_special_rows(quant):
    # all-zero rows, a row whose groups are zero but one, signed zeros, a row
    # spanning many decades (E2M1 zeros and subnormal E4M3 codes)
    M, H = 6, 512
    wl = wlmod.Workload("q_special", R=2, M=M, H=H)
    g = torch.Generator().manual_seed(3)
    x0 = torch.randn(M, H, generator=g)
    x1 = torch.randn(M, H, generator=g)
    res = torch.randn(M, H, generator=g)
    x0[0], x1[0], res[0] = 0.0, 0.0, -0.0
    x0[1], x1[1], res[1] = 0.0, -0.0, 0.0
    x0[1, 300] = 5.0
    x0[2] = torch.logspace(-30, 3, H) * torch.where(torch.arange(H) % 3 == 0, -1.0, 1.0)
    x1[2], res[2] = 0.0, 0.0
    xs = [x0.to(torch.bfloat16), x1.to(torch.bfloat16)]
    res = res.to(torch.bfloat16)
    w = (1.0 + 0.1 * torch.randn(H, generator=g)).to(torch.bfloat16)
    for path in ("one", "two"):
        _check(_run(wl, xs, res, w, quant, path, True), _oracle(wl, xs, res, w, quant, True),
               f"special/q{quant}/{path}")


def test_token_quant_equals_arrms_fused_fp8():
    # ARRMS_QUANT_FP8_TOKEN is arrms_fused with ARRMS_FP8
    wl = wlmod.FP8_GEMMA.with_(M=96, mirror=True)
    xs, res, w = wlmod.make_inputs(wl, seed=2)
    a = gu.run_hip(wl, xs, res, w)
    dev = torch.device("cuda")
    xd = [x.to(dev) for x in xs]
    rd, wd = res.to(dev), w.to(dev)
    out = torch.empty(wl.M, wl.H, dtype=torch.float16, device=dev)
    rout = torch.empty_like(out)
    q = torch.empty(wl.M, wl.H, dtype=torch.uint8, device=dev)
    sc = torch.empty(wl.M, dtype=torch.float32, device=dev)
    arrms.arrms_fused_quant(xd, rd, wd, out, rout, q, sc, eps=wl.eps, flags=wl.flags & ~oracle.FP8,
                            quant=arrms.QUANT_FP8_TOKEN)
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_bits(q), a["fp8"])
    assert np.array_equal(gu.host_bits(sc), a["scale"])
    assert np.array_equal(gu.host_bits(out), a["out"])


@pytest.mark.parametrize("quant", [2, 3], ids=["fp8group", "mxfp4"])
def test_group_quant_graph_replay(quant):
    # one captured call per path, replayed with new inputs copied into the
    # captured buffers and poisoned outputs, each replay against the oracle
    dev = torch.device("cuda")
    wl = wlmod.Workload("q_graph", R=3, M=200, H=2048, dtype="fp16", gemma=True, w_mean=0.0)
    arrms.arrms_reserve_staging(0)
    xs0, res0, w0 = wlmod.make_inputs(wl, seed=0)
    xd = [x.to(dev) for x in xs0]
    rd, wd = res0.to(dev), w0.to(dev)
    qshape, _, sshape, sdt = _shapes(quant, wl.M, wl.H)
    bufs, graphs = {}, {}
    for path in ("one", "two"):
        b = {"out": torch.empty(wl.M, wl.H, dtype=torch.float16, device=dev),
             "rout": torch.empty(wl.M, wl.H, dtype=torch.float16, device=dev),
             "q": torch.empty(qshape, dtype=torch.uint8, device=dev),
             "sc": torch.empty(sshape, dtype=sdt, device=dev)}
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            arrms.arrms_fused_quant(xd, rd, wd, b["out"], b["rout"], b["q"], b["sc"], eps=wl.eps,
                                    flags=wl.flags | PATHS[path], quant=quant, stream=s)
        torch.cuda.current_stream().wait_stream(s)
        bufs[path], graphs[path] = b, g
    for step in range(3):
        xs, res, w = wlmod.make_inputs(wl, seed=20 + step)
        for d, h in zip(xd, xs):
            d.copy_(h)
        rd.copy_(res)
        wd.copy_(w)
        want = _oracle(wl, xs, res, w, quant, True)
        for path in ("one", "two"):
            b = bufs[path]
            for t in b.values():
                gu.poison_(t)
            torch.cuda.synchronize()
            print(f"group-quant graph replay quant={quant} path={path} step={step}", flush=True)
            graphs[path].replay()
            torch.cuda.synchronize()
            got = {"out": gu.host_bits(b["out"]), "residual_out": gu.host_bits(b["rout"]),
                   "fp8": gu.host_bits(b["q"]),
                   "scale": gu.host_bits(b["sc"]) if sdt == torch.uint8 else gu.host_bits(b["sc"])}
            _check(got, want, f"graph/q{quant}/{path}/{step}")
