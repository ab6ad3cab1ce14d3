"""Pins of the oracle's adapter merge ("QLoRA, explained", Quality loss at merge time): bf16 of
W~ + s B A with one rounding.

The rounding is checked against an independent exact-rational rounding (Fraction arithmetic and a
search over neighbouring bf16 values) on random values and on constructed ties; the formula against
exact rational sums on tiny matrices; the layout with one-hot factors (a transposed B or A moves
the update to another element); and the identity B = 0.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import to_bf16_bits


def _bits(rng, shape, sigma):
    return to_bf16_bits((rng.standard_normal(shape) * sigma).astype(np.float32))


def _exact_bf16_round(v: Fraction) -> int:
    """bf16 bits of the exact rational v, round to nearest, ties to even: the two bf16 neighbours
    of v are found from its binary exponent and compared exactly."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = -v if v < 0 else v
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    # a in [1, 2): bf16 steps are 2^-7 there
    lo_m = int(a * 128)                      # floor
    lo = Fraction(lo_m, 128)
    hi = lo + Fraction(1, 128)
    d_lo, d_hi = a - lo, hi - a
    if d_lo < d_hi or (d_lo == d_hi and lo_m % 2 == 0):
        m = lo_m
    else:
        m = lo_m + 1
    if m == 256:                             # carried into the next binade
        m, e = 128, e + 1
    bits = ((e + 127) << 7) | (m - 128)
    return sign | bits


def test_rounding_matches_exact_rationals_on_random_values():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(4000) * np.exp(rng.uniform(-20, 20, 4000))
    got = oracle.bf16_bits_from_f64(x)
    for xi, gi in zip(x, got):
        assert int(gi) == _exact_bf16_round(Fraction(float(xi)))


@pytest.mark.parametrize("base", [1.0, -1.0, 0.75, 3.0, 2.0 ** -100])
def test_rounding_ties_go_to_even(base):
    # base is a bf16 value; ulp is the bf16 spacing at base; base + (k + 1/2) ulp are ties
    import math
    ex = math.frexp(abs(base))[1]
    ulp = Fraction(2) ** (ex - 8)
    b = Fraction(base)
    sgn = 1 if base > 0 else -1
    went_down = went_up = False
    for k in range(4):
        t = b + sgn * (k + Fraction(1, 2)) * ulp
        got = int(oracle.bf16_bits_from_f64(np.array([float(t)]))[0])
        assert got == _exact_bf16_round(t)
        assert got & 1 == 0                       # the even neighbour
        lower = _exact_bf16_round(b + sgn * k * ulp)
        went_down |= got == lower
        went_up |= got != lower
        for v in (t + ulp / 1024, t - ulp / 1024):
            assert int(oracle.bf16_bits_from_f64(np.array([float(v)]))[0]) == _exact_bf16_round(v)
    assert went_down and went_up                  # ties to even, not ties away or toward zero


def test_merge_equals_exact_rational_sum():
    rng = np.random.default_rng(6)
    n, k, r, s = 5, 7, 3, 2.0
    w, a, b = _bits(rng, (n, k), 0.05), _bits(rng, (r, k), 0.3), _bits(rng, (n, r), 0.3)
    got = oracle.merge(w, a, b, s)
    W, A, B = (oracle.f32_from_bf16_bits(t) for t in (w, a, b))
    for i in range(n):
        for j in range(k):
            v = Fraction(float(W[i, j])) + Fraction(s) * sum(Fraction(float(B[i, t])) * Fraction(float(A[t, j]))
                                                            for t in range(r))
            assert int(got[i, j]) == _exact_bf16_round(v)


def test_zero_adapter_returns_the_dequantised_weight():
    rng = np.random.default_rng(7)
    w = _bits(rng, (16, 64), 0.02)
    a = _bits(rng, (4, 64), 0.3)
    b = np.zeros((16, 4), dtype=np.uint16)
    assert np.array_equal(oracle.merge(w, a, b, 2.0), w)


def test_one_hot_factors_touch_one_element():
    n, k, r = 6, 8, 2
    w = np.zeros((n, k), dtype=np.uint16)
    a = np.zeros((r, k), dtype=np.uint16)
    b = np.zeros((n, r), dtype=np.uint16)
    a[1, 5] = to_bf16_bits(np.float32([0.5]))[0]
    b[3, 1] = to_bf16_bits(np.float32([0.25]))[0]
    out = oracle.merge(w, a, b, 4.0)
    want = np.zeros((n, k), dtype=np.uint16)
    want[3, 5] = to_bf16_bits(np.float32([0.5]))[0]      # 4 * 0.25 * 0.5
    assert np.array_equal(out, want)
