"""Pins of the oracle's per-group FP8 and MXFP4 outputs (CPU only).

The pages name these quant forms of the fused op without defining them; the
oracle reads per-group FP8 as the per-token steps on groups of 128 columns
and MXFP4 as OCP Microscaling Formats v1.0 (blocks of 32, E8M0 scale
2^(floor(log2 amax) - 2), E2M1 elements, RNE, saturating). These tests fix
that reading by things other than the oracle's code: the E2M1 value table
searched by exact comparison (fmt_ref), closed-form scale codes, per-group
FP8 reducing to the already pinned per-token step on each group, an
independent exact-rational MX quantiser applied to the oracle's own T
output, power-of-two scaling invariance and hand-placed exact values.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from all_reduce_residual_rank_amd import workloads as wlmod
from tests import fmt_ref

TORCH_T = {oracle.BF16: torch.bfloat16, oracle.FP16: torch.float16}


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def values(a, dt):
    return fmt_ref.bf16_value(a) if dt == oracle.BF16 else fmt_ref.fp16_value(a)


# ---- the E2M1 element format ---------------------------------------------

def test_e2m1_encoder_matches_table_search():
    # every E2M1 value, every midpoint, and points one fp32 ulp either side, both signs
    t = fmt_ref.E2M1_VALUES
    pts = list(t) + [(a + b) / 2 for a, b in zip(t[:-1], t[1:])] + [6.5, 7.0, 8.0, 1e6, 3.0e38]
    v = np.array(pts, dtype=np.float32)
    v = np.concatenate([v, np.nextafter(v, np.float32(np.inf)), np.nextafter(v, np.float32(0))])
    v = np.concatenate([v, -v])
    got = oracle.e2m1_from_float(v)
    want = fmt_ref.e2m1_bits(v.astype(np.float64))
    assert np.array_equal(got, want)


def test_e2m1_dense_random_and_specials():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(200000) * 3).astype(np.float32)
    assert np.array_equal(oracle.e2m1_from_float(v), fmt_ref.e2m1_bits(v.astype(np.float64)))
    got = oracle.e2m1_from_float(np.array([0.0, -0.0, np.inf, -np.inf], dtype=np.float32))
    assert list(got) == [0x0, 0x8, 0x7, 0xF]


# ---- per-group FP8 -----------------------------------------------------------

@pytest.mark.parametrize("dt", [oracle.BF16, oracle.FP16])
@pytest.mark.parametrize("gemma", [False, True])
def test_group_fp8_is_per_token_quant_of_each_group(dt, gemma):
    # groups of 128 columns: each group's bytes and scale are the per-token step
    # (pinned in test_oracle_fused) applied to that group of the T output
    H = 512
    wl = wlmod.Workload("g", R=3, M=6, H=H, dtype={0: "bf16", 1: "fp16"}[dt], gemma=gemma,
                        w_mean=0.0 if gemma else 1.0, row_scale=(0.1, 10.0))
    xs, res, w = wlmod.make_inputs(wl, seed=4)
    flags = dt | (oracle.GEMMA if gemma else 0)
    o = oracle.fused([bits(x) for x in xs], bits(res), bits(w), 1e-6, flags | oracle.FP8_GROUP)
    assert o["fp8"].shape == (6, H) and o["scale"].shape == (6, H // 128)
    for g in range(H // 128):
        q, sc = oracle.quant(o["out"][:, g * 128:(g + 1) * 128], dt)
        assert np.array_equal(q, o["fp8"][:, g * 128:(g + 1) * 128])
        assert np.array_equal(sc, o["scale"][:, g])


def test_group_fp8_with_one_group_equals_per_token():
    wl = wlmod.Workload("g1", R=4, M=9, H=128, dtype="fp16", gemma=True, w_mean=0.0)
    xs, res, w = wlmod.make_inputs(wl, seed=2)
    args = ([bits(x) for x in xs], bits(res), bits(w), 1e-6)
    a = oracle.fused(*args, oracle.FP16 | oracle.GEMMA | oracle.FP8_GROUP)
    b = oracle.fused(*args, oracle.FP16 | oracle.GEMMA | oracle.FP8)
    assert np.array_equal(a["fp8"], b["fp8"])
    assert np.array_equal(a["scale"][:, 0], b["scale"])
    assert np.array_equal(a["out"], b["out"])


def test_group_fp8_zero_group():
    # a row whose first group is all zero: scale 0 and signed-zero codes there
    H = 256
    x = torch.zeros(1, H)
    x[0, 128:] = torch.linspace(-3, 3, 128)
    res = torch.zeros(1, H)
    res[0, :128] = -0.0
    w = torch.ones(H)
    o = oracle.fused([bits(x.to(torch.bfloat16))], bits(res.to(torch.bfloat16)),
                     bits(w.to(torch.bfloat16)), 1e-6, oracle.BF16 | oracle.FP8_GROUP)
    assert o["scale"][0, 0] == 0.0 and o["scale"][0, 1] > 0
    assert np.all((o["fp8"][0, :128] & 0x7F) == 0)


def test_group_and_mx_need_whole_groups():
    x = [np.zeros((2, 96), dtype=np.uint16)]
    with pytest.raises(ValueError):
        oracle.fused(x, x[0], np.zeros(96, dtype=np.uint16), 1e-6, oracle.BF16 | oracle.FP8_GROUP)
    y = [np.zeros((2, 48), dtype=np.uint16)]
    with pytest.raises(ValueError):
        oracle.fused(y, y[0], np.zeros(48, dtype=np.uint16), 1e-6, oracle.BF16 | oracle.MXFP4)


# ---- MXFP4 ---------------------------------------------------------------------

def _mx_reference(y: np.ndarray):
    """Independent MXFP4 of T values y [M][H] (float64), written from the spec:
    exponent by exact comparison with powers of two, elements by table search."""
    M, H = y.shape
    codes = np.zeros((M, H), dtype=np.uint8)
    scales = np.zeros((M, H // 32), dtype=np.uint8)
    for m in range(M):
        for b in range(H // 32):
            blk = y[m, b * 32:(b + 1) * 32]
            amax = Fraction(float(np.max(np.abs(blk))))
            if amax == 0:
                e = -127
            else:
                k = 0
                while Fraction(2) ** (k + 1) <= amax:
                    k += 1
                while Fraction(2) ** k > amax:
                    k -= 1
                e = max(-127, min(127, k - 2))
            scales[m, b] = e + 127
            for j in range(32):
                v = Fraction(float(blk[j])) / Fraction(2) ** e
                c = fmt_ref.nearest_fraction(v, fmt_ref.E2M1_VALUES, "sat") if v != 0 else 0
                if np.signbit(blk[j]):
                    c |= 0x8
                codes[m, b * 32 + j] = c
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.FP16])
@pytest.mark.parametrize("gemma", [False, True])
def test_mxfp4_matches_independent_reference(dt, gemma):
    H = 256
    wl = wlmod.Workload("mx", R=2, M=5, H=H, dtype={0: "bf16", 1: "fp16"}[dt], gemma=gemma,
                        w_mean=0.0 if gemma else 1.0, x_sigma=2.0, row_scale=(0.01, 100.0))
    xs, res, w = wlmod.make_inputs(wl, seed=6)
    flags = dt | (oracle.GEMMA if gemma else 0)
    o = oracle.fused([bits(x) for x in xs], bits(res), bits(w), 1e-6, flags | oracle.MXFP4)
    assert o["fp8"].shape == (5, H // 2) and o["scale"].shape == (5, H // 32)
    q, sc = _mx_reference(values(o["out"], dt))
    assert np.array_equal(sc, o["scale"])
    assert np.array_equal(q, o["fp8"])


def _mx_of_row(vals, dt=oracle.BF16):
    """MXFP4 of one row whose T output is exactly vals (R=1, zero residual,
    unit weight, eps chosen so that rstd = 1 exactly)."""
    vals = np.asarray(vals, dtype=np.float64)
    H = vals.size
    ss = float(np.sum(vals * vals))
    eps = 1.0 - ss / H
    assert 0 <= eps and np.float32(eps) == eps
    T = TORCH_T[dt]
    x = bits(torch.tensor(vals, dtype=torch.float64).reshape(1, H).to(T))
    z = bits(torch.zeros(1, H, dtype=T))
    w = bits(torch.ones(H, dtype=T))
    o = oracle.fused([x], z, w, float(eps), dt | oracle.MXFP4)
    assert np.array_equal(values(o["out"], dt)[0], vals)   # y = h exactly
    return o


def test_mxfp4_exact_values_and_scale_closed_form():
    # block 0: amax 6 * 2^-4 -> X = 2^-4 (code 123): elements are exact E2M1 values
    e2m1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6] * 4) * 2.0 ** -4
    e2m1[1::2] *= -1
    # block 1: amax 1.0 -> X = 2^-2 (code 125); values 1, 0.5, ... land on 4, 2, ...
    b1 = np.array([1.0, 0.5, 0.25, 0.125] * 8) * np.array([1, -1] * 16)
    vals = np.concatenate([e2m1, b1])
    o = _mx_of_row(vals)
    assert list(o["scale"][0]) == [123, 125]
    codes = np.zeros(64, dtype=np.uint8)
    codes[0::2] = o["fp8"][0] & 0xF
    codes[1::2] = o["fp8"][0] >> 4
    assert np.array_equal(fmt_ref.e2m1_value(codes[:32]) * 2.0 ** -4, e2m1)
    assert np.array_equal(fmt_ref.e2m1_value(codes[32:]) * 2.0 ** -2, b1)


def test_mxfp4_ties_go_to_even():
    # X = 2^-2 (amax 1): y/X = 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4,
    # 5 -> 4 (the even neighbour each time)
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = np.array(ties + [4.0] + [0.0] * 24) * 0.25
    o = _mx_of_row(vals)
    assert o["scale"][0, 0] == 125
    c = np.zeros(32, dtype=np.uint8)
    c[0::2] = o["fp8"][0] & 0xF
    c[1::2] = o["fp8"][0] >> 4
    assert list(fmt_ref.e2m1_value(c[:8])) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 4.0]


@pytest.mark.parametrize("k", [-3, -1, 1, 5])
def test_mxfp4_power_of_two_scaling(k):
    # scaling every input by 2^k scales y by 2^k only if rstd is unchanged;
    # instead scale the weights: y = h * w * rstd scales by 2^k exactly, so the
    # scale codes move by k and the element codes stay
    wl = wlmod.Workload("mxs", R=2, M=4, H=128, row_scale=(0.1, 10.0))
    xs, res, w = wlmod.make_inputs(wl, seed=9)
    args = ([bits(x) for x in xs], bits(res))
    a = oracle.fused(*args, bits(w), 1e-6, oracle.BF16 | oracle.MXFP4)
    b = oracle.fused(*args, bits(w * 2.0 ** k), 1e-6, oracle.BF16 | oracle.MXFP4)
    assert np.array_equal(a["fp8"], b["fp8"])
    assert np.array_equal(a["scale"].astype(int) + k, b["scale"].astype(int))


def test_mxfp4_block_max_lands_on_4_or_6():
    # amax / X lies in [4, 8): its code is 4.0 or (saturated or rounded) 6.0
    wl = wlmod.Workload("mxm", R=4, M=8, H=256, dtype="fp16", x_sigma=2.0)
    xs, res, w = wlmod.make_inputs(wl, seed=1)
    o = oracle.fused([bits(x) for x in xs], bits(res), bits(w), 1e-6, oracle.FP16 | oracle.MXFP4)
    y = values(o["out"], oracle.FP16)
    c = np.zeros(y.shape, dtype=np.uint8)
    c[:, 0::2] = o["fp8"] & 0xF
    c[:, 1::2] = o["fp8"] >> 4
    for m in range(8):
        for b in range(256 // 32):
            j = b * 32 + int(np.argmax(np.abs(y[m, b * 32:(b + 1) * 32])))
            assert abs(fmt_ref.e2m1_value(c[m, j])) in (4.0, 6.0)


def test_mxfp4_zero_block():
    vals = np.zeros(32)
    vals[0] = -0.0
    o = _mx_of_row(np.concatenate([vals, np.full(32, 0.5)]))
    assert o["scale"][0, 0] == 0                       # all-zero block: 2^-127
    assert np.all(o["fp8"][0, :16] & 0x77 == 0)        # +-0 codes
