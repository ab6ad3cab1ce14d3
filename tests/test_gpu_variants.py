"""GPU parity of the codebook and blocksize variants and of dequantisation without double
quantisation ("QLoRA, explained", A toy run; Double quantisation): every packed index, absmax and
bf16 output bit-exact against the oracle.

Inputs: Student-t weights (heavy tails, like the 70B-shaped workload) with constructed blocks in
front: an all-zero block, a block holding every decision midpoint of the codebook exactly (as fp32,
with scale 1, so the fp32 midpoints that are exact are ties and the rest are within 2^-25 of one),
a block on the fast path's bin edges, and a block whose scale is below 2^-100. The element count
leaves the last workgroup (4096 values) partly empty wherever the blocksize allows.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import bits_from_dev, dev, log, to_dev
from oracle import toy

pytestmark = pytest.mark.gpu

BOOKS = {"nf4": oracle.codebook, "fp4": toy.fp4_codebook, "int4": toy.int4_codebook}


def _inputs(book, bs, seed):
    codes = BOOKS[book]().astype(np.float64)
    unit = max(bs, 64)
    n = 4096 * 24 + (unit * 3 if unit < 4096 else 0)
    g = wl.rng_for("stream", 300 + seed, "w")
    w = (g.standard_t(4, size=n) * 0.015).astype(np.float32)
    mids = ((codes[:-1] + codes[1:]) / 2).astype(np.float32)
    edges = (-1.0 + np.arange(1, 256) / 128.0).astype(np.float32)
    special = [np.zeros(bs, np.float32)]
    b = np.resize(np.concatenate([[1.0], mids, -mids]).astype(np.float32), bs)
    b[0] = 1.0
    special.append(b)
    e = np.resize(edges, bs)
    e[0] = -1.0
    special.append(e)
    t = (np.resize(mids, bs) * np.float32(1e-35)).astype(np.float32)
    t[0] = np.float32(3e-35)
    special.append(t)
    s = np.concatenate(special)
    w[: s.size] = s
    return w


def _gpu_quant(w, book, bs):
    import torch
    import bit_nf4_quantised_amd as q
    packed = torch.empty(w.size // 2, dtype=torch.uint8, device=dev())
    absmax = torch.empty(w.size // bs, dtype=torch.float32, device=dev())
    q.q4_quantize(to_dev(w), book, bs, packed, absmax)
    torch.cuda.synchronize()
    return packed.cpu().numpy(), absmax.cpu().numpy()


def _gpu_dequant(packed, n, book, bs, **scales):
    import torch
    import bit_nf4_quantised_amd as q
    out = torch.empty(n, dtype=torch.int16, device=dev())
    q.q4_dequant(to_dev(packed), n, book, bs, out, **{k: to_dev(v) for k, v in scales.items()})
    torch.cuda.synchronize()
    return bits_from_dev(out)


@pytest.mark.parametrize("bs", [16, 32, 64, 128, 512, 2048, 4096])
@pytest.mark.parametrize("book", ["nf4", "fp4", "int4"])
def test_variant_matches_oracle(book, bs):
    log(f"[variants] {book} blocksize {bs}")
    codes = BOOKS[book]()
    w = _inputs(book, bs, bs)
    packed, absmax = _gpu_quant(w, book, bs)
    ref_p, ref_a = oracle.quantize_with(w, codes, bs)
    assert np.array_equal(absmax.view(np.uint32), ref_a.view(np.uint32)), "absmax differs"
    bad = np.flatnonzero(packed != ref_p)
    assert bad.size == 0, f"{bad.size} packed bytes differ, first at byte {bad[:5]}"
    # dequantisation with the fp32 scales (no double quantisation)
    got = _gpu_dequant(ref_p, w.size, book, bs, absmax=ref_a)
    assert np.array_equal(got, oracle.dequant_blocks(ref_p, ref_a, codes, bs, w.size))
    # and with double-quantised scales
    sq, c2 = oracle.double_quant(ref_a)
    got = _gpu_dequant(ref_p, w.size, book, bs, scale_q=sq, scale_c2=c2)
    assert np.array_equal(got, oracle.dequant_blocks(ref_p, oracle.dequant_scales(sq, c2), codes, bs, w.size))


def test_nf4_blocksize_64_equals_the_nf4_kernels():
    import torch
    import bit_nf4_quantised_amd as q
    w = _inputs("nf4", 64, 1)[: 4096 * 24]
    packed, absmax = _gpu_quant(w, "nf4", 64)
    qw = q.quantize_weight(to_dev(w).reshape(1536, 64))
    torch.cuda.synchronize()
    assert np.array_equal(packed, qw.packed.cpu().numpy())
    out = torch.empty(w.size, dtype=torch.int16, device=dev())
    q.nf4_dequant(qw, out)
    got = _gpu_dequant(packed, w.size, "nf4", 64, scale_q=qw.scale_q.cpu().numpy(),
                       scale_c2=qw.scale_c2.cpu().numpy())
    assert np.array_equal(got, bits_from_dev(out))


@pytest.mark.parametrize("book,bs", [("fp4", 256), ("int4", 16)])
def test_full_stream_matrix_sampled(book, bs):
    # the benchmark's shape (one 4096 x 14336 stream matrix): sampled blocks against the oracle
    w = wl.stream_weight(0)
    packed, absmax = _gpu_quant(w, book, bs)
    codes = BOOKS[book]()
    flat = w.reshape(-1)
    rng = np.random.default_rng(bs)
    blocks = np.unique(np.concatenate([[0, flat.size // bs - 1], rng.integers(0, flat.size // bs, 3000)]))
    for b in blocks:
        vals = flat[b * bs:(b + 1) * bs]
        rp, ra = oracle.quantize_with(vals, codes, bs)
        assert absmax[b] == ra[0]
        assert np.array_equal(packed[b * bs // 2:(b + 1) * bs // 2], rp)
    got = _gpu_dequant(packed, flat.size, book, bs, absmax=absmax).reshape(-1, bs)
    for b in blocks[:500]:
        ref = oracle.dequant_blocks(packed[b * bs // 2:(b + 1) * bs // 2], absmax[b:b + 1], codes, bs, bs)
        assert np.array_equal(got[b], ref)
