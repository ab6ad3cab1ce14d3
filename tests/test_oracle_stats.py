"""The oracle's quantiser reproduces the statistics the page prints for its numpy toy run.

"QLoRA, explained", A toy run: how much does NF4 lose, and can LoRA win it back? A wrong index,
a dropped scale, a mis-ordered codebook or a wrong tie rule moves these numbers far outside the
page's printed digits. Gaussian figures at blocksize 64 match to every printed digit; the
Student-t and blocksize 4096 figures depend on the draw, so they carry a sampling tolerance.
"""
import json
import os

import numpy as np

import oracle
from oracle import toy

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "toy_statistics.json")))
BOOKS = {"nf4": oracle.codebook, "fp4": toy.fp4_codebook, "int4": toy.int4_codebook}


def _gauss():
    return np.random.default_rng(0).normal(0, 0.02, 2 ** 20)


def test_gaussian_blocksize64():
    w = _gauss()
    for name, fn in BOOKS.items():
        e = toy.relative_mse(w, fn(), 64)
        assert round(100 * e, 3) == G["gaussian_bs64_pct"][name], name
        assert round(-10 * np.log10(e), 2) == G["gaussian_bs64_sqnr_db"][name], name


def test_student_t5():
    t = np.random.default_rng(0).standard_t(5, 2 ** 20) * 0.02 * np.sqrt(3 / 5)
    for name, fn in BOOKS.items():
        e = 100 * toy.relative_mse(t, fn(), 64)
        want = G["student_t5_bs64_pct"][name]
        assert abs(e - want) <= 0.01 * want, (name, e, want)
    # the ordering the page reports: NF4 < FP4 < INT4, with INT4 hurt most by the heavy tail
    e = {n: toy.relative_mse(t, fn(), 64) for n, fn in BOOKS.items()}
    assert e["nf4"] < e["fp4"] < e["int4"]


def test_blocksize_trend():
    w = _gauss()
    got = {bs: 100 * toy.relative_mse(w, None, bs) for bs in (16, 64, 4096)}
    want = G["nf4_by_blocksize_pct"]
    assert abs(got[16] - want["16"]) <= 0.002
    assert abs(got[64] - want["64"]) <= 0.003
    assert abs(got[4096] - want["4096"]) <= 0.02
    assert got[16] < got[64] < got[4096]


def test_residual_capture():
    w = np.random.default_rng(0).normal(0, 0.02, (1024, 1024))
    cap = toy.residual_capture(w, [16, 64, 256])
    want = G["residual_capture_1024x1024_pct"]
    assert round(100 * cap[0], 2) == want["16"]
    assert round(100 * cap[1], 1) == want["64"]
    assert round(100 * cap[2], 1) == want["256"]
