"""Pins of the oracle's plain rank all-reduce (step O1 alone; CPU only).

Fixed by: the exact-integer generator of ROCm/aiter PR #5807 (its reproducer
checks exact integer sums), hand-worked rounding cases whose answers follow
from the formats alone (a tie kept by fp32 but not by bf16 steps, a sum that
fp32 accumulation rounds away before the final rounding, a rank-order
witness), signed zeros, overflow to infinity and gradual underflow. A
plausible slip -- rounding to T after every add, accumulating in fp64, a
reversed or pairwise rank order, starting from +0 -- fails one of them.
"""
import numpy as np
import pytest
import torch

import oracle
from all_reduce_residual_rank_amd import workloads as wlmod
from tests import fmt_ref

TORCH_T = {oracle.BF16: torch.bfloat16, oracle.FP16: torch.float16, oracle.FP32: torch.float32}


def bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.float32:
        return t.contiguous().numpy().copy()
    return t.contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def vals(vs, dt) -> list[np.ndarray]:
    """One single-element rank array per value (exactly representable in T)."""
    return [bits(torch.tensor([v], dtype=TORCH_T[dt])) for v in vs]


def as_float(a: np.ndarray, dt: int) -> np.ndarray:
    if dt == oracle.FP32:
        return a.astype(np.float64)
    return fmt_ref.bf16_value(a) if dt == oracle.BF16 else fmt_ref.fp16_value(a)


@pytest.mark.parametrize("dt_name", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("R", [1, 2, 4, 8])
def test_exact_integer_generator(dt_name, R):
    # PR #5807 reproducer: rank r holds ((i(r+1) + seed(r+3)) % 31) - 15; every
    # partial sum is a small integer, so the result is the integer sum exactly.
    dt = wlmod.DT_CODE[dt_name]
    n = 4096 + 8 * 37
    for seed in (1, 7, 106):
        xs = [bits(x.reshape(-1)) for x in wlmod.exact_integer_inputs(R, 1, n, seed, dt_name)]
        idx = np.arange(n)
        want = sum(((idx * (r + 1) + seed * (r + 3)) % 31) - 15 for r in range(R))
        got = oracle.rank_sum(xs, dt)
        assert np.array_equal(as_float(got, dt), want.astype(np.float64))


def test_fp32_rank_order_witness():
    # fp32: 1 + 2^-24 is a tie between 1 and 1 + 2^-23 and goes to 1 (even);
    # left to right the small terms vanish one by one, added first they meet.
    tiny = 2.0 ** -24
    got = oracle.rank_sum(vals([1.0, tiny, tiny], oracle.FP32), oracle.FP32)
    assert got[0] == np.float32(1.0)
    got = oracle.rank_sum(vals([tiny, tiny, 1.0], oracle.FP32), oracle.FP32)
    assert got[0] == np.float32(1.0 + 2.0 ** -23)


def test_bf16_rounds_once_after_the_fp32_sum():
    # 1 + 2^-8 + 2^-8 = 1 + 2^-7 exactly in fp32 -> bf16 0x3f81. Rounding to
    # bf16 after each add would hit the tie 1 + 2^-8 twice and stay at 1.0.
    got = oracle.rank_sum(vals([1.0, 2.0 ** -8, 2.0 ** -8], oracle.BF16), oracle.BF16)
    assert got[0] == 0x3F81


def test_bf16_accumulates_in_fp32_not_exactly():
    # 1 + 2^-8 + 2^-33: fp32 drops 2^-33 (below half an ulp of 1), leaving the
    # bf16 tie 1 + 2^-8, which goes to 1.0 (0x3f80). The exact sum lies above
    # the tie and would round to 0x3f81.
    got = oracle.rank_sum(vals([1.0, 2.0 ** -8, 2.0 ** -33], oracle.BF16), oracle.BF16)
    assert got[0] == 0x3F80


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.FP16, oracle.FP32])
def test_signed_zeros(dt):
    # the accumulator starts at x_0: all -0 stays -0; any +0 makes +0
    got = oracle.rank_sum(vals([-0.0, -0.0, -0.0], dt), dt)
    assert np.signbit(as_float(got, dt)[0]) and as_float(got, dt)[0] == 0.0
    got = oracle.rank_sum(vals([-0.0, 0.0, -0.0], dt), dt)
    assert not np.signbit(as_float(got, dt)[0])
    got = oracle.rank_sum(vals([-0.0], dt), dt)
    assert np.signbit(as_float(got, dt)[0])


def test_overflow_and_underflow():
    # bf16 max + bf16 max exceeds fp32 max -> +inf
    bmax = fmt_ref.bf16_value(np.array([0x7F7F], dtype=np.uint16))[0]
    got = oracle.rank_sum(vals([bmax, bmax], oracle.BF16), oracle.BF16)
    assert got[0] == 0x7F80
    # fp16 65504 + 65504 = 131008 is finite in fp32, infinite in fp16
    got = oracle.rank_sum(vals([65504.0, 65504.0], oracle.FP16), oracle.FP16)
    assert got[0] == 0x7C00
    got = oracle.rank_sum(vals([-65504.0, -65504.0], oracle.FP16), oracle.FP16)
    assert got[0] == 0xFC00
    # fp32 max + fp32 max -> inf; max + (-max) -> +0
    fmax = float(np.finfo(np.float32).max)
    got = oracle.rank_sum(vals([fmax, fmax], oracle.FP32), oracle.FP32)
    assert np.isinf(got[0]) and got[0] > 0
    # fp16 subnormals add exactly: 2^-24 * 3
    got = oracle.rank_sum(vals([2.0 ** -24] * 3, oracle.FP16), oracle.FP16)
    assert got[0] == 0x0003
    # bf16 subnormal region: 2^-133 + 2^-133 = 2^-132, exact
    got = oracle.rank_sum(vals([2.0 ** -133, 2.0 ** -133], oracle.BF16), oracle.BF16)
    assert as_float(got, oracle.BF16)[0] == 2.0 ** -132


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.FP16, oracle.FP32])
def test_matches_fused_residual_out_with_negative_zero_residual(dt):
    # a + (-0) = a for every a (also -0), so the fused epilogue's residual_out
    # with an all -0 residual is this rank sum: the two definitions agree.
    wl = wlmod.Workload("t", R=4, M=5, H=64, dtype={0: "bf16", 1: "fp16", 2: "fp32"}[dt],
                        row_scale=(0.1, 10.0))
    xs, _, w = wlmod.make_inputs(wl, seed=3)
    xs = [bits(x) for x in xs]
    res = bits(torch.full((5, 64), -0.0, dtype=TORCH_T[dt]))
    o = oracle.fused(xs, res, bits(w), 1e-6, dt)
    assert np.array_equal(oracle.rank_sum(xs, dt), o["residual_out"])


def test_sum_cases_follow_the_sweep():
    # the flattened sweep's sizes: 16-byte packs, both aligned and ragged tiles
    for dt in ("bf16", "fp16", "fp32"):
        cases = wlmod.sum_cases(dt)
        assert len({c.numel for c in cases}) == len(cases)
        assert all(c.nbytes % 16 == 0 for c in cases)
        tails = [c for c in cases if (c.nbytes // 16) % 512]
        assert tails and len(tails) < len(cases)
