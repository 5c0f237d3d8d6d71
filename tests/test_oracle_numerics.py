"""Pins for the oracle's number formats against exact rational arithmetic."""
from fractions import Fraction

import numpy as np
import pytest

from oracle.numerics import bf16_to_f64, f64_to_f16_bits, f16_bits_to_f64

# every finite, non-negative fp16 value, as exact fractions, in increasing order
_POS = np.arange(0, 0x7C00, dtype=np.uint16)
_POS_F = [Fraction(float(v)) for v in _POS.view(np.float16).astype(np.float64)]
_MAXF16 = Fraction(65504)
_HALF_ULP_TOP = Fraction(2 ** 15) * Fraction(2 ** -10) / 2  # half ulp at the top binade


def _exact_round_f16(v: float) -> int:
    """Nearest fp16 (ties to even mantissa) by exhaustive search over the binade table."""
    f = Fraction(v)
    sign = 0x8000 if f < 0 or (f == 0 and np.signbit(v)) else 0
    a = abs(f)
    if a >= _MAXF16 + _HALF_ULP_TOP:
        return sign | 0x7C00
    lo, hi = 0, len(_POS_F) - 1
    while lo < hi:  # first index with value >= a
        mid = (lo + hi) // 2
        if _POS_F[mid] < a:
            lo = mid + 1
        else:
            hi = mid
    if _POS_F[lo] == a:
        return sign | lo
    below, above = lo - 1, lo
    if above >= len(_POS_F):
        return sign | below
    db, da = a - _POS_F[below], _POS_F[above] - a
    if db < da:
        return sign | below
    if da < db:
        return sign | above
    return sign | (below if below % 2 == 0 else above)


def test_f16_matches_exact_rounding_random():
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.standard_normal(3000) * 0.05,
        rng.standard_normal(1000) * 1e-5,          # subnormal range
        rng.uniform(-70000, 70000, 500),           # overflow boundary
        np.exp(rng.uniform(-25, 11, 1000)),
    ])
    got = f64_to_f16_bits(vals)
    for v, g in zip(vals.tolist(), got.tolist()):
        assert g == _exact_round_f16(v), (v, hex(g))


def test_f16_halfway_ties_to_even_and_no_double_rounding():
    # exact halfway between 1 and 1+2^-10 rounds to even (1.0)
    assert f64_to_f16_bits(1.0 + 2.0 ** -11) == 0x3C00
    # halfway between 1+2^-10 and 1+2^-9 rounds to even (1+2^-9)
    assert f64_to_f16_bits(1.0 + 3 * 2.0 ** -11) == 0x3C02
    # just above halfway must round up; a float32 detour would round it to 1.0
    assert f64_to_f16_bits(1.0 + 2.0 ** -11 + 2.0 ** -40) == 0x3C01
    # smallest subnormal and its halfway point
    assert f64_to_f16_bits(2.0 ** -24) == 0x0001
    assert f64_to_f16_bits(2.0 ** -25) == 0x0000
    assert f64_to_f16_bits(3 * 2.0 ** -25) == 0x0002
    # overflow threshold: 65520 is halfway between 65504 and 2^16 -> inf
    assert f64_to_f16_bits(65519.99) == 0x7BFF
    assert f64_to_f16_bits(65520.0) == 0x7C00


def test_f16_roundtrip_all_finite():
    bits = np.arange(0, 0x7C00, dtype=np.uint16)
    assert np.array_equal(f64_to_f16_bits(f16_bits_to_f64(bits)), bits)


def test_bf16_decode_exact():
    # 0x3F80 = 1.0, 0xC000 = -2.0, 0x3C23 = 0x3C230000 as float32
    assert bf16_to_f64(np.array([0x3F80, 0xC000], dtype=np.uint16)).tolist() == [1.0, -2.0]
    v = bf16_to_f64(np.array([0x3C23], dtype=np.uint16))[0]
    assert v == float(np.array([0x3C230000], dtype=np.uint32).view(np.float32)[0])
