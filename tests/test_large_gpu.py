"""Tensors past 4 GiB, on a GPU: row byte offsets above 2^32 in the row kernel,
the two-stage chunk loop over hundreds of staging chunks, and the flat sum's
element index beyond 2^31. Inputs are drawn on the device; the oracle checks
sampled rows (each row's outputs depend only on that row's inputs and the
weights) and sampled spans of the flat sum, to the usual bars.
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

R, M, H = 2, 350_000, 6144          # one [M][H] bf16 tensor: 4.30 GB
ROW_BYTES = H * 2
PATHS = {"one": 16, "two": 32}


def _rows():
    edge = (1 << 32) // ROW_BYTES  # the row that straddles byte 2^32
    rng = np.random.default_rng(7)
    fixed = [0, 1, 2, M // 2, edge - 1, edge, edge + 1, M - 2, M - 1]
    return sorted(set(fixed) | set(int(r) for r in rng.integers(0, M, 9)))


def _device_inputs(dev):
    g = torch.Generator(device=dev).manual_seed(11)
    xs = [torch.randn(M, H, device=dev, dtype=torch.bfloat16, generator=g) for _ in range(R)]
    res = torch.randn(M, H, device=dev, dtype=torch.bfloat16, generator=g)
    w = (1.0 + 0.1 * torch.randn(H, device=dev, generator=g)).to(torch.bfloat16)
    return xs, res, w


@pytest.mark.parametrize("path", ["one", "two"])
def test_fused_past_4gib(path):
    dev = torch.device("cuda")
    assert M * ROW_BYTES > (1 << 32)
    xs, res, w = _device_inputs(dev)
    out = gu.poison_(torch.empty(M, H, dtype=torch.bfloat16, device=dev))
    rout = gu.poison_(torch.empty(M, H, dtype=torch.bfloat16, device=dev))
    q = gu.poison_(torch.empty(M, H, dtype=torch.uint8, device=dev))
    sc = gu.poison_(torch.empty(M, dtype=torch.float32, device=dev))
    flags = arrms.DTYPE_BF16 | arrms.FP8 | PATHS[path]
    print(f"large case R={R} M={M} H={H} bf16 fp8+mirror path={path}", flush=True)
    arrms.arrms_fused(xs, res, w, out, rout, q, sc, eps=1e-6, flags=flags)
    torch.cuda.synchronize()
    rows = torch.tensor(_rows(), device=dev)
    got = {"out": gu.host_bits(out[rows]), "residual_out": gu.host_bits(rout[rows]),
           "fp8": gu.host_bits(q[rows]), "scale": gu.host_bits(sc[rows])}
    want = oracle.fused([gu.host_bits(x[rows]) for x in xs], gu.host_bits(res[rows]), gu.host_bits(w),
                        1e-6, oracle.FP8 | wlmod.DT_CODE["bf16"], want_out=True)
    gu.compare(got, want, "bf16", label=f"large/{path}")
    del xs, res, w, out, rout, q, sc
    torch.cuda.empty_cache()


def test_sum_past_2g_elements():
    dev = torch.device("cuda")
    n = M * H
    assert n > (1 << 31)
    g = torch.Generator(device=dev).manual_seed(12)
    xs = [torch.randn(n, device=dev, dtype=torch.bfloat16, generator=g) for _ in range(4)]
    out = gu.poison_(torch.empty(n, dtype=torch.bfloat16, device=dev))
    print(f"large sum R=4 n={n} bf16", flush=True)
    arrms.arrms_allreduce_sum(xs, out, flags=arrms.DTYPE_BF16)
    torch.cuda.synchronize()
    span = 4096
    # element 2^30 starts byte 2^31, element 2^31 starts byte 2^32
    starts = [0, (1 << 30) - span // 2, (1 << 31) - span // 2, n // 2, n - span]
    for s in starts:
        want = oracle.rank_sum([gu.host_bits(x[s:s + span]) for x in xs], wlmod.DT_CODE["bf16"])
        got = gu.host_bits(out[s:s + span])
        assert np.array_equal(got, want), f"sum span at {s}"
    del xs, out
    torch.cuda.empty_cache()
