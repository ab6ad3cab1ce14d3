"""Pins of the oracle's blockwise quantiser, nibble packing, double quantisation and dequantisation.

Each check compares the oracle with something other than itself: the page's worked example
("QLoRA, explained", Worked example), exact rational brute force written independently here,
torch's float8_e4m3fn and bfloat16 casts, and the page's storage arithmetic.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- independent brute force helpers
def brute_nearest(block, codes):
    """First argmin over codes of the exact |w/c - q_i| (Fractions); the zero code if c == 0."""
    fr = [Fraction(float(v)) for v in block]
    c = max(abs(v) for v in fr)
    qs = [Fraction(float(q)) for q in codes]
    if c == 0:
        return [qs.index(0)] * len(fr), c
    out = []
    for v in fr:
        d = [abs(v / c - q) for q in qs]
        out.append(d.index(min(d)))
    return out, c


def brute_e4m3_nearest(ratio: Fraction):
    """Nearest E4M3 value in [0, 1] to an exact ratio; ties to the even code."""
    vals = [oracle.e4m3_value(c) for c in range(0x39)]
    d = [abs(ratio - v) for v in vals]
    best = min(d)
    cands = [i for i, x in enumerate(d) if x == best]
    if len(cands) == 1:
        return cands[0]
    return [c for c in cands if c % 2 == 0][0]


# ---------------------------------------------------------------- worked example
def test_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    w = np.array(ex["block"], dtype=np.float32)
    idx, c = oracle.quantize_blocks(w, blocksize=8)
    assert list(idx[0]) == ex["indices"]
    assert c[0] == np.float32(ex["absmax"])
    q = oracle.codebook().astype(np.float64)
    c64 = float(c[0])
    norm = w.astype(np.float64) / c64
    assert [round(v, 3) for v in norm] == ex["normalised"]
    assert [round(q[i], 4) for i in idx[0]] == ex["codes"]
    rec = q[idx[0]] * c64
    assert [round(v, 4) for v in rec] == ex["reconstructed"]
    assert [round(abs(a - b), 4) for a, b in zip(rec, w.astype(np.float64))] == ex["abs_error"]
    # the block's absmax element maps to code -1 or +1, so it comes back exactly
    assert rec[3] == float(w[3])


# ---------------------------------------------------------------- nearest code: brute force
def _adversarial_blocks():
    q = oracle.codebook().astype(np.float64)
    mids = (q[:-1] + q[1:]) / 2
    blocks = []
    rng = np.random.default_rng(7)
    # midpoint ties: with a power-of-two scale c, c * m_i is a float32 whenever m_i is one
    for i, m in enumerate(mids):
        if np.float32(m) == m:
            c = np.float32(0.5)
            b = rng.normal(0, 0.1, 64).astype(np.float32)
            b = np.clip(b, -0.49, 0.49).astype(np.float32)
            b[0] = c
            b[1] = np.float32(c * m)                      # exactly on the midpoint -> lower index
            b[2] = np.nextafter(np.float32(c * m), np.float32(1))   # just above -> upper index
            b[3] = np.nextafter(np.float32(c * m), np.float32(-1))  # just below -> lower index
            blocks.append(b)
    blocks.append(np.zeros(64, np.float32))                              # all zero
    z = np.zeros(64, np.float32); z[5] = -0.0; z[9] = np.float32(-3e-3); blocks.append(z)
    s = np.zeros(64, np.float32); s[17] = np.float32(1e-30); blocks.append(s)   # single nonzero
    e = np.full(64, np.float32(0.01)); e[::2] = np.float32(-0.01); blocks.append(e)  # +-c
    t = np.full(64, np.float32(-0.0)); t[0] = np.float32(2.0); blocks.append(t)
    sub = (rng.normal(0, 1, 64) * 1e-40).astype(np.float32); blocks.append(sub)  # subnormal
    return blocks


def test_nearest_code_matches_brute_force():
    codes = oracle.codebook()
    rng = np.random.default_rng(1)
    blocks = _adversarial_blocks()
    for _ in range(40):
        blocks.append(rng.standard_normal(64).astype(np.float32) * np.float32(rng.uniform(1e-3, 3)))
    for _ in range(10):
        b = rng.standard_t(3, 64).astype(np.float32)
        blocks.append(b)
    w = np.concatenate(blocks)
    idx, c = oracle.quantize_blocks(w)
    for bi, b in enumerate(blocks):
        want, cw = brute_nearest(b, codes)
        assert list(idx[bi]) == want, bi
        assert Fraction(float(c[bi])) == cw


def test_tie_goes_to_lower_index():
    q = oracle.codebook().astype(np.float64)
    m7 = (q[7] + q[8]) / 2
    assert np.float32(m7) == m7
    b = np.zeros(64, np.float32); b[0] = 1.0; b[1] = np.float32(m7)
    idx, _ = oracle.quantize_blocks(b)
    assert idx[0, 1] == 7 and idx[0, 0] == 15


def test_other_codebooks_match_brute_force():
    from oracle import toy
    rng = np.random.default_rng(3)
    for codes in (toy.int4_codebook(), toy.fp4_codebook()):
        w = rng.standard_normal(64 * 8).astype(np.float32)
        idx, _ = oracle.quantize_blocks(w, 64, codes)
        for bi in range(8):
            want, _ = brute_nearest(w[bi * 64:(bi + 1) * 64], codes)
            assert list(idx[bi]) == want


def test_requantise_is_idempotent():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal(64 * 64) * 0.02).astype(np.float32)
    idx, c = oracle.quantize_blocks(w)
    q = oracle.codebook()
    rec = (q[idx] * c[:, None]).astype(np.float32)
    idx2, c2 = oracle.quantize_blocks(rec.reshape(-1))
    assert np.array_equal(idx, idx2)
    assert np.array_equal(c, c2)


def test_pack_order_and_roundtrip():
    idx = np.array([1, 2, 15, 0, 7, 8], np.uint8)
    p = oracle.pack_nibbles(idx)
    assert list(p) == [0x12, 0xF0, 0x78]
    rng = np.random.default_rng(4)
    i2 = rng.integers(0, 16, 1000).astype(np.uint8)
    assert np.array_equal(oracle.unpack_nibbles(oracle.pack_nibbles(i2)), i2)


def test_quantize_rejects_ragged():
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros(65, np.float32))


# ---------------------------------------------------------------- 8-bit floats and double quant
def test_e4m3_decode_matches_torch():
    codes = [c for c in range(256) if c & 0x7F != 0x7F]
    t = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([float(oracle.e4m3_value(c)) for c in codes])
    assert np.array_equal(t, mine)
    unit = oracle.e4m3_unit_values()
    assert unit.size == 57 and unit[0] == 0 and unit[-1] == 1.0 and np.all(np.diff(unit) > 0)


def test_double_quant_matches_brute_force():
    rng = np.random.default_rng(5)
    nb = 256 * 3 + 77                                 # partial last group
    c1 = np.abs(rng.standard_normal(nb) * 0.06).astype(np.float32)
    c1[256:512] = 0                                   # an all-zero group -> c2 = 0, codes 0
    c1[600] = np.float32(1e-12)                       # far below the smallest E4M3 step
    c1[601] = 0
    codes, c2 = oracle.double_quant(c1)
    assert c2.shape == (4,) and c2.dtype == np.float32 and codes.dtype == np.uint8
    for g in range(4):
        assert c2[g] == c1[g * 256:(g + 1) * 256].max()
    for i in range(nb):
        g = i // 256
        if c2[g] == 0:
            assert codes[i] == 0
            continue
        want = brute_e4m3_nearest(Fraction(float(c1[i])) / Fraction(float(c2[g])))
        assert codes[i] == want, i


def test_double_quant_ties_go_to_even():
    unit = oracle.e4m3_unit_values()
    c1 = []
    for j in range(56):
        c1.append((unit[j] + unit[j + 1]) / 2)          # exact midpoints with c2 = 1
    c1 = np.array(c1 + [1.0], np.float32)
    assert np.array_equal(c1[:-1].astype(np.float64), (unit[:-1] + unit[1:]) / 2)
    codes, c2 = oracle.double_quant(c1)
    assert c2[0] == 1.0
    for j in range(56):
        assert codes[j] == (j if j % 2 == 0 else j + 1)


def test_double_quant_matches_torch_cast_when_c2_is_one():
    """With c2 = 1 the ratio is c1 itself, a float32, so torch's round-to-nearest-even float8 cast
    is an independent reference."""
    rng = np.random.default_rng(6)
    c1 = rng.uniform(0, 1, 4096).astype(np.float32)
    c1[::256] = 1.0
    codes, c2 = oracle.double_quant(c1)
    assert np.all(c2 == 1.0)
    t = torch.from_numpy(c1).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, t)


def test_dequant_scales_exact_product():
    rng = np.random.default_rng(8)
    codes = rng.integers(0, 0x39, 512).astype(np.uint8)
    c2 = np.abs(rng.standard_normal(2)).astype(np.float32)
    got = oracle.dequant_scales(codes, c2)
    for i in range(512):
        exact = oracle.e4m3_value(int(codes[i])) * Fraction(float(c2[i // 256]))
        assert float(exact) == float(Fraction(float(exact)))     # fits float64 exactly
        assert got[i] == np.float32(float(exact))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    bits[::3] = (bits[::3] & 0xFFFF0000) | 0x8000                  # exact ties
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    x = x[np.abs(x) < 3e38]                                        # no rounding to infinity
    mine = oracle.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_dequant_matches_library_composition():
    """w~ = bf16(fl32(q[idx] * fl32(e4m3(code) * c2))) rebuilt with torch casts and float32 tensors."""
    rng = np.random.default_rng(10)
    w = (rng.standard_normal(64 * 300) * 0.02).astype(np.float32)
    packed, c1 = oracle.quantize(w)
    codes, c2 = oracle.double_quant(c1)
    got = oracle.dequant(packed, codes, c2, w.size)
    idx = torch.from_numpy(oracle.unpack_nibbles(packed).astype(np.int64))
    q = torch.from_numpy(oracle.codebook())
    e4 = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32)
    c2t = torch.from_numpy(c2).repeat_interleave(256)[: codes.size]
    c1p = e4 * c2t
    ref = (q[idx].view(-1, 64) * c1p[:, None]).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(got, ref.view(np.uint16).reshape(-1))


def test_dequant_of_zero_block_is_positive_zero():
    w = np.zeros(128, np.float32); w[64:] = np.linspace(-1, 1, 64, dtype=np.float32)
    packed, c1 = oracle.quantize(w)
    codes, c2 = oracle.double_quant(c1)
    out = oracle.dequant(packed, codes, c2, 128)
    assert np.all(out[:64] == 0)


# ---------------------------------------------------------------- storage arithmetic
def test_storage_bits_match_pages():
    g = json.load(open(os.path.join(GOLDEN, "toy_statistics.json")))["bits_per_param"]
    assert round(oracle.storage_bits(64), 3) == g["bs64_dq"]
    assert round(oracle.storage_bits(64, False) - oracle.storage_bits(64), 3) == g["dq_saving"]
    assert oracle.storage_bits(16, False) == g["bs16_no_dq"]
    assert round(oracle.storage_bits(16), 3) == g["bs16_dq"]
    assert oracle.storage_bits(64, False) - 4 == g["bs64_fp32_scales_overhead"]


# ---------------------------------------------------------------- codebook and blocksize variants
@pytest.mark.parametrize("book,bs", [("fp4", 16), ("int4", 256), ("nf4", 32), ("fp4", 4096)])
def test_dequant_blocks_matches_torch_composition(book, bs):
    """bf16(fl32(q[idx] * absmax)) rebuilt with float32 torch tensors and torch's bf16 cast, for
    the toy's other codebooks and other blocksizes, with fp32 scales (no double quantisation)."""
    from oracle import toy
    codes = {"nf4": oracle.codebook(), "fp4": toy.fp4_codebook(), "int4": toy.int4_codebook()}[book]
    rng = np.random.default_rng(bs)
    w = (rng.standard_normal(8192) * 0.03).astype(np.float32)
    w[:bs] = 0.0                                                   # one all-zero block
    packed, absmax = oracle.quantize_with(w, codes, bs)
    got = oracle.dequant_blocks(packed, absmax, codes, bs, w.size)
    idx = torch.from_numpy(oracle.unpack_nibbles(packed).astype(np.int64))
    q = torch.from_numpy(codes)
    ref = (q[idx].view(-1, bs) * torch.from_numpy(absmax)[:, None]).to(torch.bfloat16)
    assert np.array_equal(got, ref.view(torch.int16).numpy().view(np.uint16).reshape(-1))
    assert np.all(got[:bs] == 0)


def test_dequant_blocks_reduces_to_the_nf4_path():
    """NF4, blocksize 64, double-quantised scales: the generic dequantisation is the two-level one."""
    rng = np.random.default_rng(21)
    w = (rng.standard_normal(64 * 520) * 0.02).astype(np.float32)
    packed, c1 = oracle.quantize_with(w, oracle.codebook(), 64)
    assert np.array_equal(packed, oracle.quantize(w)[0])
    codes, c2 = oracle.double_quant(c1)
    got = oracle.dequant_blocks(packed, oracle.dequant_scales(codes, c2), oracle.codebook(), 64, w.size)
    assert np.array_equal(got, oracle.dequant(packed, codes, c2, w.size))


@pytest.mark.parametrize("bs", [16, 32, 128, 1024])
def test_quantize_with_blocksizes_matches_brute_force(bs):
    from oracle import toy
    rng = np.random.default_rng(bs + 1)
    for codes in (oracle.codebook(), toy.fp4_codebook(), toy.int4_codebook()):
        w = rng.standard_normal(2 * bs).astype(np.float32)
        packed, absmax = oracle.quantize_with(w, codes, bs)
        idx = oracle.unpack_nibbles(packed)
        for bi in range(2):
            want, c = brute_nearest(w[bi * bs:(bi + 1) * bs], codes)
            assert list(idx[bi * bs:(bi + 1) * bs]) == want
            assert Fraction(float(absmax[bi])) == c
