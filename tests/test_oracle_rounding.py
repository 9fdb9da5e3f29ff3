"""Pins of the oracle's number-format conversions (CPU only).

The oracle's encoders are checked against (a) a nearest-value table search
written from the format definitions (tests/fmt_ref.py), and (b) independent
library casts: torch's float32 -> bfloat16 and float32 -> float8_e4m3fn,
numpy's float64 -> float16 (a direct, single rounding).
"""
import numpy as np
import pytest
import torch

import oracle
from tests import fmt_ref


def _structured_f32(low_halves=(0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF)):
    """Every (sign, exponent, top-7 fraction bits) pattern with chosen low halves."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    rng = np.random.default_rng(1234)
    lows = list(low_halves) + list(rng.integers(0, 1 << 16, size=4))
    bits = (hi[:, None] | np.array(lows, dtype=np.uint32)[None, :]).ravel()
    f = bits.view(np.float32)
    return f[np.isfinite(f)]


def test_bf16_matches_torch_cast_on_float32():
    f = _structured_f32()
    got = oracle.bf16_from_double(f.astype(np.float64))
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_bf16_matches_table_on_doubles_near_ties():
    # Doubles at, and one double-ulp either side of, every bf16 midpoint in a wide
    # exponent range: a float32 detour would round some of these twice.
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 0x7F7F, size=20000)
    lo = fmt_ref.BF16_VALUES[codes]
    hi = fmt_ref.BF16_VALUES[codes + 1]
    mid = lo + (hi - lo) / 2
    v = np.concatenate([mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf), lo, hi])
    v = np.concatenate([v, -v, rng.standard_normal(20000) * 10.0 ** rng.uniform(-40, 38, 20000)])
    got = oracle.bf16_from_double(v)
    assert np.array_equal(got, fmt_ref.bf16_bits(v))


def test_bf16_special_values():
    inf_edge = fmt_ref.BF16_VALUES[-1] + (fmt_ref.BF16_VALUES[-1] - fmt_ref.BF16_VALUES[-2]) / 2
    v = np.array([0.0, -0.0, np.inf, -np.inf, inf_edge, np.nextafter(inf_edge, 0), 2.0 ** -133,
                  2.0 ** -134, 3 * 2.0 ** -134])
    got = oracle.bf16_from_double(v)
    assert list(got) == [0x0000, 0x8000, 0x7F80, 0xFF80, 0x7F80, 0x7F7F, 0x0001, 0x0000, 0x0002]
    assert oracle.bf16_from_double(np.array([np.nan]))[0] & 0x7FFF > 0x7F80


def test_fp16_matches_numpy_direct_cast():
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 0x7BFF, size=30000)
    lo = fmt_ref.FP16_VALUES[codes]
    hi = fmt_ref.FP16_VALUES[codes + 1]
    mid = lo + (hi - lo) / 2
    v = np.concatenate([mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf), lo,
                        rng.standard_normal(30000) * 10.0 ** rng.uniform(-9, 5, 30000),
                        [65504.0, 65519.99, 65520.0, 70000.0, 2.0 ** -24, 2.0 ** -25,
                         np.nextafter(2.0 ** -25, 1), 1e-9]])
    v = np.concatenate([v, -v])
    got = oracle.fp16_from_double(v)
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)
    assert np.array_equal(got, fmt_ref.fp16_bits(v))


def test_e4m3_matches_table_everywhere_and_torch_in_range():
    f = _structured_f32(low_halves=(0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF))
    # the e4m3 ties sit at fraction bit 19 of float32: add patterns that hit them exactly
    hi = np.arange(1 << 12, dtype=np.uint32) << 20
    extra = (hi[:, None] | np.array([0x80000, 0x7FFFF, 0x80001, 0, 0xFFFFF], dtype=np.uint32)[None, :]).ravel()
    extra = extra.view(np.float32)
    f = np.concatenate([f, extra[np.isfinite(extra)], -extra[np.isfinite(extra)]])
    got = oracle.e4m3_from_float(f)
    assert np.array_equal(got, fmt_ref.e4m3_bits(f.astype(np.float64)))
    inr = np.abs(f) <= 448.0
    want = torch.from_numpy(f[inr]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got[inr], want)


def test_e4m3_saturation_and_specials():
    v = np.array([448.0, 463.99, 464.0, 1e6, np.inf, -1e6, -0.0, 0.0, 2.0 ** -9, 2.0 ** -10,
                  3 * 2.0 ** -10, 2.0 ** -6], dtype=np.float32)
    got = oracle.e4m3_from_float(v)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x01, 0x00, 0x02, 0x08]
    assert oracle.e4m3_from_float(np.array([np.nan], dtype=np.float32))[0] & 0x7F == 0x7F


def test_tables_decode_like_libraries():
    # the references themselves: decoded tables agree with library decoders
    b = np.arange(0x7F80, dtype=np.uint32)
    assert np.array_equal(fmt_ref.BF16_VALUES, (b[: 0x7F80] << 16).view(np.float32)[: 0x7F80].astype(np.float64))
    h = np.arange(0x7C00, dtype=np.uint16)
    assert np.array_equal(fmt_ref.FP16_VALUES, h.view(np.float16).astype(np.float64))
    q = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(fmt_ref.E4M3_VALUES, q)
    assert fmt_ref.E4M3_VALUES[-1] == 448.0


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.FP16])
def test_quant_rows_scale_is_fp32_division(dt):
    rng = np.random.default_rng(3)
    y = rng.standard_normal((5, 64))
    bits = oracle.bf16_from_double(y) if dt == oracle.BF16 else oracle.fp16_from_double(y)
    bits = bits.reshape(5, 64)
    vals = fmt_ref.bf16_value(bits) if dt == oracle.BF16 else fmt_ref.fp16_value(bits)
    q, sc = oracle.quant(bits, dt)
    amax = np.abs(vals).max(axis=1).astype(np.float32)
    assert np.array_equal(sc, amax / np.float32(448.0))
    want = fmt_ref.e4m3_bits((vals.astype(np.float32) / sc[:, None]).astype(np.float64))
    assert np.array_equal(q, want)
    # the row maximum encodes to +-448
    for m in range(5):
        j = np.argmax(np.abs(vals[m]))
        assert q[m, j] & 0x7F == 0x7E


# Each exported function of liboracle.so, with a test in this suite that pins it
# against something other than the oracle itself (format tables, library casts,
# closed forms, brute force).
PINNED_EXPORTS = {
    "oracle_fused_rows": "test_oracle_fused.py (closed forms, exact-rational brute force, torch fp64 RMSNorm)",
    "oracle_rank_sum": "test_oracle_rank_sum.py (rank-order witness, exact integers, torch fp32 sums)",
    "oracle_quant_rows": "test_oracle_fused.py / test_oracle_group_quant.py (E4M3 table, amax/448)",
    "orc_bf16_from_double_n": "test_bf16_matches_torch_cast_on_float32 and the table search",
    "orc_fp16_from_double_n": "the numpy float64 -> float16 cast and the table search",
    "orc_e4m3_from_float_n": "the torch float8_e4m3fn cast and the table search",
    "orc_e2m1_from_float_n": "test_oracle_group_quant.py (E2M1 table search)",
}


def test_every_oracle_export_is_pinned():
    """The oracle library exports exactly the functions listed above: a new or
    leftover export without a pin fails here."""
    import subprocess
    oracle._load()
    out = subprocess.run(["nm", "-D", "--defined-only", oracle._LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if len(ln.split()) == 3 and ln.split()[1] == "T"}
    assert exported == set(PINNED_EXPORTS)
