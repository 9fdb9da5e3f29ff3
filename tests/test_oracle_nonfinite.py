"""Pins of the oracle's handling of non-finite values (CPU only).

The pages define nothing for NaN or infinity. The reading taken: IEEE
arithmetic throughout, plus three rules -- a maximum over |y| (per-token or
per-group FP8, MXFP4 block) is NaN when any y it covers is NaN; every NaN
encodes as the E4M3 code 0x7F, with no sign; in an MXFP4 block whose scale is
the NaN code a NaN element is 0x7 and the others +-6's code with y's sign.

The pins use what the arithmetic fixes independently of the oracle's code:
weights are shared by all rows and do not enter rstd, so a non-finite weight
changes only its own column of y, and every other column must equal the run
with a finite weight there; a non-finite h makes the row's rstd, and so every
y of that row, NaN.
"""
import numpy as np

import oracle
from tests import fmt_ref

R, M, H = 2, 3, 256
DT = oracle.BF16


def _inputs(seed=4):
    rng = np.random.default_rng(seed)
    f = lambda *s: fmt_ref.bf16_bits(rng.standard_normal(s).astype(np.float32))
    xs = [f(M, H) for _ in range(R)]
    res = f(M, H)
    w = fmt_ref.bf16_bits((1.0 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    return xs, res, w


def _isnan_bf16(b):
    return (b & 0x7FFF) > 0x7F80


def _val(b):
    return fmt_ref.bf16_value(b)


def _run(xs, res, w, quant):
    return oracle.fused(xs, res, w, 1e-6, DT | quant, want_out=True)


NAN_BF16 = 0x7FC0
INF_BF16 = 0x7F80


def _with_weight(w, j, bits):
    w2 = w.copy()
    w2[j] = bits
    return w2


def test_e4m3_nan_code_has_no_sign():
    with np.errstate(invalid="ignore"):
        v = np.array([np.nan, -np.nan, np.float32(np.inf) - np.float32(np.inf)], dtype=np.float32)
    v[1] = -np.abs(v[1])
    assert np.signbit(v[1])
    assert list(oracle.e4m3_from_float(v)) == [0x7F, 0x7F, 0x7F]


def test_nan_weight_per_token():
    xs, res, w = _inputs()
    j = 37
    base = _run(xs, res, _with_weight(w, j, 0x3F80), oracle.FP8)
    got = _run(xs, res, _with_weight(w, j, NAN_BF16), oracle.FP8)
    assert np.array_equal(got["residual_out"], base["residual_out"])
    assert _isnan_bf16(got["out"][:, j]).all()
    keep = np.arange(H) != j
    assert np.array_equal(got["out"][:, keep], base["out"][:, keep])
    assert np.isnan(got["scale"]).all()
    assert (got["fp8"] == 0x7F).all()


def test_nan_weight_per_group():
    xs, res, w = _inputs()
    j = 37  # group 0 of 2
    base = _run(xs, res, _with_weight(w, j, 0x3F80), oracle.FP8_GROUP)
    got = _run(xs, res, _with_weight(w, j, NAN_BF16), oracle.FP8_GROUP)
    assert np.isnan(got["scale"][:, 0]).all()
    assert (got["fp8"][:, :128] == 0x7F).all()
    assert np.array_equal(got["scale"][:, 1], base["scale"][:, 1])
    assert np.array_equal(got["fp8"][:, 128:], base["fp8"][:, 128:])


def test_nan_weight_mxfp4():
    xs, res, w = _inputs()
    j = 37  # block 1 (columns 32..63)
    base = _run(xs, res, _with_weight(w, j, 0x3F80), oracle.MXFP4)
    got = _run(xs, res, _with_weight(w, j, NAN_BF16), oracle.MXFP4)
    assert (got["scale"][:, 1] == 0xFF).all()
    other = [b for b in range(H // 32) if b != 1]
    assert np.array_equal(got["scale"][:, other], base["scale"][:, other])
    nib = np.stack([got["fp8"] & 0xF, got["fp8"] >> 4], axis=-1).reshape(M, H)
    base_nib = np.stack([base["fp8"] & 0xF, base["fp8"] >> 4], axis=-1).reshape(M, H)
    assert (nib[:, j] == 0x7).all()
    cols = [c for c in range(32, 64) if c != j]
    sign = np.where(_val(base["out"][:, cols]) < 0, 0x8, 0x0)
    assert np.array_equal(nib[:, cols], sign | 0x7)
    outside = np.r_[0:32, 64:H]
    assert np.array_equal(nib[:, outside], base_nib[:, outside])


def test_nan_in_residual_poisons_its_row_only():
    xs, res, w = _inputs()
    res2 = res.copy()
    res2[2, 200] = NAN_BF16
    base = _run(xs, res, w, oracle.FP8)
    got = _run(xs, res2, w, oracle.FP8)
    assert _isnan_bf16(got["residual_out"][2, 200])
    keep = np.ones((M, H), bool)
    keep[2, 200] = False
    assert np.array_equal(got["residual_out"][keep], base["residual_out"][keep])
    assert _isnan_bf16(got["out"][2]).all()
    assert np.array_equal(got["out"][:2], base["out"][:2])
    assert np.isnan(got["scale"][2]) and np.array_equal(got["scale"][:2], base["scale"][:2])
    assert (got["fp8"][2] == 0x7F).all()
    assert np.array_equal(got["fp8"][:2], base["fp8"][:2])
    mx = _run(xs, res2, w, oracle.MXFP4)
    assert (mx["scale"][2] == 0xFF).all() and (mx["fp8"][2] == 0x77).all()


def test_infinite_weight():
    xs, res, w = _inputs()
    j = 5
    base = _run(xs, res, _with_weight(w, j, 0x3F80), oracle.FP8)
    got = _run(xs, res, _with_weight(w, j, INF_BF16), oracle.FP8)
    h = _val(got["residual_out"][:, j])
    assert np.all(h != 0)
    assert np.array_equal(_val(got["out"][:, j]), np.where(h > 0, np.inf, -np.inf))
    keep = np.arange(H) != j
    assert np.array_equal(got["out"][:, keep], base["out"][:, keep])
    # amax = inf: finite y / inf = +-0 (sign of y); inf / inf is NaN -> 0x7F
    assert np.isinf(got["scale"]).all()
    assert (got["fp8"][:, j] == 0x7F).all()
    y = _val(got["out"][:, keep])
    want = np.where(np.signbit(y), 0x80, 0x00)
    assert np.array_equal(got["fp8"][:, keep], want)
    mx = _run(xs, res, _with_weight(w, j, INF_BF16), oracle.MXFP4)
    assert (mx["scale"][:, 0] == 0xFF).all()
    nib = np.stack([mx["fp8"] & 0xF, mx["fp8"] >> 4], axis=-1).reshape(M, H)
    yb = _val(mx["out"][:, :32])
    assert np.array_equal(nib[:, :32], np.where(np.signbit(yb), 0x8, 0x0) | 0x7)
