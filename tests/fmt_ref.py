"""Independent references for the number formats, used to pin the oracle.

Nothing here calls the oracle or the HIP library. Each format is described
only by the list of its finite non-negative values, decoded from the bit
layout with plain integer arithmetic; rounding to the format is "pick the
nearest value in that list, ties to the code with an even last bit", done by
exact comparison. That is the definition of round-to-nearest-even, written
out as a table search rather than as bit manipulation.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def _decode_table(ebits: int, mbits: int, bias: int, top_code: int) -> np.ndarray:
    """Values of codes 0..top_code (non-negative, finite) of a binary format."""
    codes = np.arange(top_code + 1, dtype=np.int64)
    e = codes >> mbits
    m = codes & ((1 << mbits) - 1)
    vals = np.where(e == 0,
                    np.ldexp(m.astype(np.float64), 1 - bias - mbits),
                    np.ldexp((m + (1 << mbits)).astype(np.float64), (e - bias - mbits).astype(np.int64)))
    return vals


# bf16: 8 exponent bits, 7 fraction bits, bias 127; 0x7F7F is the largest finite.
BF16_VALUES = _decode_table(8, 7, 127, 0x7F7F)
# fp16: 5 exponent bits, 10 fraction bits, bias 15; 0x7BFF = 65504.
FP16_VALUES = _decode_table(5, 10, 15, 0x7BFF)
# E4M3 "fn": 4 exponent bits, 3 fraction bits, bias 7; 0x7E = 448 (0x7F is NaN).
E4M3_VALUES = _decode_table(4, 3, 7, 0x7E)
# E2M1 (OCP MX FP4): 2 exponent bits, 1 fraction bit, bias 1; 0x7 = 6, no inf/NaN.
E2M1_VALUES = _decode_table(2, 1, 1, 0x7)


def nearest_code(v: np.ndarray, table: np.ndarray, overflow: str) -> np.ndarray:
    """Round finite doubles v to the table's format; returns codes (int64, sign in bit 'sign').

    overflow='inf': beyond max + half an ulp gives the infinity code (max+1);
    overflow='sat': saturate to the max code. Returns magnitude codes and a
    sign array separately to stay format-agnostic.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    hi = np.searchsorted(table, a, side="left")          # table[hi-1] < a <= table[hi]
    hi_c = np.minimum(hi, len(table) - 1)
    lo_c = np.maximum(hi - 1, 0)
    exact = table[hi_c] == a
    d_lo = a - table[lo_c]                                # exact (Sterbenz) for adjacent values
    d_hi = table[hi_c] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi_c % 2 == 0))
    code = np.where(exact, hi_c, np.where(pick_hi, hi_c, lo_c))
    top = len(table) - 1
    beyond = hi > top                                      # a > max finite
    if overflow == "inf":
        ulp_top = table[top] - table[top - 1]
        half = table[top] + ulp_top / 2
        # at exactly max + half ulp the even neighbour is the (odd-coded) max's successor: infinity
        code = np.where(beyond & (a >= half), top + 1, np.where(beyond, top, code))
    else:
        code = np.where(beyond, top, code)
    return code


def bf16_bits(v) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    c = nearest_code(v, BF16_VALUES, "inf").astype(np.uint16)   # 0x7F80 = inf
    return (c | np.where(np.signbit(v), 0x8000, 0).astype(np.uint16)).astype(np.uint16)


def fp16_bits(v) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    c = nearest_code(v, FP16_VALUES, "inf").astype(np.uint16)   # 0x7C00 = inf
    return (c | np.where(np.signbit(v), 0x8000, 0).astype(np.uint16)).astype(np.uint16)


def e4m3_bits(v) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    c = nearest_code(v, E4M3_VALUES, "sat").astype(np.uint8)
    return (c | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)).astype(np.uint8)


def e2m1_bits(v) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    c = nearest_code(v, E2M1_VALUES, "sat").astype(np.uint8)
    return (c | np.where(np.signbit(v), 0x8, 0).astype(np.uint8)).astype(np.uint8)


def e2m1_value(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    mag = E2M1_VALUES[b & 0x7]
    return np.where(b & 0x8, -mag, mag)


def bf16_value(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def fp16_value(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def e4m3_value(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    mag = E4M3_VALUES[np.minimum(b & 0x7F, 0x7E)]
    return np.where(b & 0x80, -mag, mag)


def nearest_fraction(x: Fraction, table: np.ndarray, overflow: str = "inf") -> int:
    """Exact-rational version of nearest_code for one value (ties to even code)."""
    a = abs(x)
    fa = float(a)
    i = int(np.searchsorted(table, fa, side="left"))
    best = None
    for c in range(max(i - 2, 0), min(i + 2, len(table))):
        d = abs(Fraction(float(table[c])) - a)
        key = (d, c % 2)
        if best is None or key < best[0]:
            best = (key, c)
    top = len(table) - 1
    if a > Fraction(float(table[top])):
        half = Fraction(float(table[top])) + (Fraction(float(table[top])) - Fraction(float(table[top - 1]))) / 2
        if overflow == "inf" and a >= half:
            return top + 1
        return top
    return best[1]
