"""Parity of the plain rank all-reduce (arrms_allreduce_sum) with the oracle's
rank sum, on a GPU, over the flattened message sweep of ROCm/aiter PR #5807
(representative sizes, the 1 MiB tile boundary and its neighbours, the
(M, 2880) rows and the (1023/1024/1025, 512) rows) in bf16, fp16 and fp32.

The bar is bit-exact. Outputs are poisoned with NaN bytes before each call and
followed by a poisoned guard region that must survive, so that both a missed
element and a write past the end of a ragged last tile show up.
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

GUARD = 256  # elements after the output that must stay untouched


def _inputs(kind, R, numel, seed, dtype):
    if kind == "int":
        return [x.reshape(-1) for x in wlmod.exact_integer_inputs(R, 1, numel, seed, dtype)]
    return wlmod.make_sum_inputs(R, numel, seed, dtype, sigma=1.0)


def _run(xs, dtype, *, inplace_rank=None):
    dev = torch.device("cuda")
    T = gu.TORCH_T[dtype]
    n = xs[0].numel()
    xd = [x.to(dev) for x in xs]
    if inplace_rank is None:
        buf = gu.poison_(torch.empty(n + GUARD, dtype=T, device=dev))
        out = buf[:n]
    else:
        out = xd[inplace_rank]
        buf = None
    arrms.arrms_allreduce_sum(xd, out, flags=wlmod.DT_CODE[dtype])
    torch.cuda.synchronize()
    if buf is not None:
        guard = gu.host_bits(buf[n:]).view(np.uint8)
        assert np.all(guard == 0xFF), "write past the end of the output"
    return gu.host_bits(out)


def _check(kind, R, numel, seed, dtype, **kw):
    print(f"sum case kind={kind} R={R} n={numel} {dtype} seed={seed} {kw}", flush=True)
    xs = _inputs(kind, R, numel, seed, dtype)
    want = oracle.rank_sum([gu.host_bits(x) for x in xs], wlmod.DT_CODE[dtype])
    got = _run(xs, dtype, **kw)
    bad = got != want
    assert not bad.any(), f"{bad.sum()} of {numel} elements differ (first at {np.argmax(bad)})"
    return got


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("kind", ["int", "normal"])
def test_sweep_sizes_r4(dtype, kind):
    for i, case in enumerate(wlmod.sum_cases(dtype)):
        _check(kind, 4, case.numel, 1 + i, dtype)


@pytest.mark.parametrize("R", [1, 2, 3, 5, 6, 7, 8])
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_rank_counts(R, dtype):
    # an aligned and a ragged message for every rank count
    for numel in (65536, 1025 * 512):
        _check("normal", R, numel, 10 + R, dtype)
        _check("int", R, numel, 20 + R, dtype)


@pytest.mark.parametrize("numel_bytes", [16, 32, 8176, 8192 + 16, 16 * 511, 16 * 513])
def test_tiny_and_single_pack_tails(numel_bytes):
    # single-lane tails: a message of one pack, and one pack either side of a tile
    for dtype in ("bf16", "fp32"):
        e = 4 if dtype == "fp32" else 2
        _check("normal", 4, numel_bytes // e, 3, dtype)


@pytest.mark.parametrize("rank", [0, 3])
def test_in_place(rank):
    for dtype in ("bf16", "fp16"):
        _check("normal", 4, 1025 * 512, 5, dtype, inplace_rank=rank)


def test_large_message_with_large_values():
    # finite fp16 inputs near the top of the range: many of the R=8 sums
    # overflow fp16 (never fp32), and the infinities must match too
    xs = [x.float().clamp(-6.0e4, 6.0e4).to(torch.float16)
          for x in wlmod.make_sum_inputs(8, 4 << 20, 9, "fp32", sigma=2.0e4)]
    want = oracle.rank_sum([gu.host_bits(x) for x in xs], 1)
    assert np.any((want & 0x7FFF) == 0x7C00)
    got = _run(xs, "fp16")
    assert np.array_equal(got, want)


def test_repeated_rank_pointers():
    dev = torch.device("cuda")
    x = wlmod.make_sum_inputs(1, 70000 * 8, 4, "bf16")[0]
    xd = x.to(dev)
    out = gu.poison_(torch.empty_like(xd))
    arrms.arrms_allreduce_sum([xd, xd, xd], out, flags=0)
    torch.cuda.synchronize()
    want = oracle.rank_sum([gu.host_bits(x)] * 3, 0)
    assert np.array_equal(gu.host_bits(out), want)


def test_graph_replay_with_changing_inputs():
    # one captured call, replayed with fresh inputs copied into the captured
    # buffers and a poisoned output, eager work and syncs between replays
    dev = torch.device("cuda")
    n = 1025 * 512
    xs0 = _inputs("int", 4, n, 1, "bf16")
    xd = [x.to(dev) for x in xs0]
    out = torch.empty(n, dtype=torch.bfloat16, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        arrms.arrms_allreduce_sum(xd, out, flags=0, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for step in range(4):
        xs = _inputs("int" if step % 2 else "normal", 4, n, 30 + step, "bf16")
        for d, h in zip(xd, xs):
            d.copy_(h)
        gu.poison_(out)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = oracle.rank_sum([gu.host_bits(x) for x in xs], 0)
        assert np.array_equal(gu.host_bits(out), want), f"replay {step}"


def test_matches_fused_residual_out():
    # the flat sum is stage 1 of the two-stage fused path: with an all -0
    # residual, the fused residual_out must equal the plain sum bit for bit
    wl = wlmod.Workload("sumcheck", R=4, M=121, H=2880, row_scale=(0.1, 10.0))
    xs, _, w = wlmod.make_inputs(wl, seed=2)
    res = torch.full((wl.M, wl.H), -0.0, dtype=torch.bfloat16)
    fused = gu.run_hip(wl, xs, res, w)
    got = _run([x.reshape(-1) for x in xs], "bf16")
    assert np.array_equal(got, fused["residual_out"].reshape(-1))
