"""Pins of the oracle's NF4 codebook against the pages, not against itself.

Sources: "QLoRA, explained", NormalFloat 4 (NF4) (construction and invariants) and Worked example
(nine codes printed to four decimals).
"""
import json
import os

import mpmath
import numpy as np
import scipy.special

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_invariants():
    q = oracle.codebook().astype(np.float64)
    assert q.shape == (16,)
    assert oracle.codebook().dtype == np.float32
    assert np.all(np.diff(q) > 0), "ascending, distinct"
    assert q[0] == -1.0 and q[-1] == 1.0, "endpoints +-1"
    assert np.all((q >= -1) & (q <= 1))
    zeros = np.flatnonzero(q == 0.0)
    assert list(zeros) == [oracle.NF4_ZERO_INDEX] == [7], "exactly one exact zero, at index 7"
    # 8 codes at or below zero and 9 at or above it: zero belongs to both halves
    assert (q <= 0).sum() == 8 and (q >= 0).sum() == 9
    # denser near zero: gaps grow outward on each side
    neg_gaps = np.diff(q[:8])[::-1]      # from zero outward
    pos_gaps = np.diff(q[7:])
    assert np.all(np.diff(neg_gaps) > 0) and np.all(np.diff(pos_gaps) > 0)


def test_printed_codes():
    """The worked example prints nine codes and their indices; 0.5626 is quoted beside them."""
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    q = oracle.codebook().astype(np.float64)
    for idx, code in zip(ex["indices"], ex["codes"]):
        assert round(q[idx], 4) == code, (idx, q[idx], code)
    assert round(q[13], 4) == 0.5626


def test_quantiles_against_high_precision():
    """The float64 evaluation agrees with a 50-digit evaluation and with scipy's ndtri, and no code
    sits near a float32 rounding boundary, so the float32 table does not depend on the routine."""
    mpmath.mp.dps = 50
    delta = (mpmath.mpf(29) / 30 + mpmath.mpf(31) / 32) / 2
    half = mpmath.mpf(1) / 2
    inv = lambda p: mpmath.sqrt(2) * mpmath.erfinv(2 * p - 1)
    top = inv(delta)
    pos = [inv(delta - i * (delta - half) / 8) / top for i in range(8)]
    neg = [-inv(delta - i * (delta - half) / 7) / top for i in range(7)]
    hp = sorted(pos + neg + [mpmath.mpf(0)])
    q32 = oracle.codebook()
    for v, c in zip(hp, q32):
        assert abs(float(v) - float(c)) <= float(np.spacing(np.float32(abs(c)))) / 2 + 1e-300
        # distance of the exact value from the fp32 rounding boundaries, in fp32 ulps
        if c != 0 and abs(c) != 1:
            ulp = mpmath.mpf(float(np.spacing(np.float32(abs(c)))))
            frac = abs(v - mpmath.mpf(float(c))) / ulp
            assert frac < mpmath.mpf("0.49"), "not within 0.01 ulp of a tie"
    # scipy's independent inverse normal gives the same float32 codes
    d = 929 / 960
    sp = sorted([scipy.special.ndtri(d - i * (d - 0.5) / 8) for i in range(8)]
                + [-scipy.special.ndtri(d - i * (d - 0.5) / 7) for i in range(7)] + [0.0])
    sp = (np.array(sp) / scipy.special.ndtri(d)).astype(np.float32)
    assert np.array_equal(sp.view(np.uint32), q32.view(np.uint32))


def test_delta_is_pinned_by_printed_codes():
    """Neighbouring readings of the tail probability fail to reproduce the printed codes, so the
    printed values do pin the construction (the readings tried: 1-1/32, 1-1/30, 16/17)."""
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))

    def book(delta):
        p = [scipy.special.ndtri(delta - i * (delta - 0.5) / 8) for i in range(8)]
        n = [-scipy.special.ndtri(delta - i * (delta - 0.5) / 7) for i in range(7)]
        return np.array(sorted(p + n + [0.0])) / scipy.special.ndtri(delta)

    def matches(delta):
        q = book(delta)
        return all(round(q[i], 4) == c for i, c in zip(ex["indices"], ex["codes"]))

    assert matches(929 / 960)
    for other in (1 - 1 / 32, 1 - 1 / 30, 16 / 17):
        assert not matches(other)
