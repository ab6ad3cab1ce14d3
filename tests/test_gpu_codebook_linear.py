"""GPU parity of the FP4 and INT4 codebooks through the adapted linear, the few-token forward, the
merge and nf4_dequant ("QLoRA, explained", A toy run, which sets NF4 beside E2M1 FP4 and an INT4
grid): a weight quantised with q4_quantize at blocksize 64 (double quantised, or keeping its fp32
absmax) and named by its codebook runs through every call that takes a weight.

Bars: the dequantisation and the merge bit-exact against the oracle; forward and backward within
the linear layer's tolerance (relative Frobenius error <= 5e-3, elementwise <= 1e-2 * max|ref|)
against the oracle's float64 linear on the oracle's own dequantised weight; with B = 0, one-hot
rows of x give rows of y equal to columns of that weight bit for bit, and one-hot rows of dY give
rows of dX equal to its rows.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import (assert_close, bf16_to_dev, bits_from_dev, dev, f64_from_bits, gpu_dequant,
                         gpu_fwd_bwd, log, to_dev)
from oracle import toy

pytestmark = pytest.mark.gpu

BOOKS = {"fp4": (1, toy.fp4_codebook), "int4": (2, toy.int4_codebook)}


def _inputs(seed, M, N, K, r):
    w = wl.weight("single", 400 + seed, N, K, "student_t4", 0.02)
    g = wl.rng_for("single", 400 + seed, "x")
    x = wl.to_bf16_bits(g.standard_normal((M, K), dtype=np.float32))
    a = wl.to_bf16_bits(g.standard_normal((r, K), dtype=np.float32) * np.float32(0.01))
    b = wl.to_bf16_bits(g.standard_normal((N, r), dtype=np.float32) * np.float32(0.01))
    dy = wl.to_bf16_bits(g.standard_normal((M, N), dtype=np.float32))
    return w, x, a, b, dy


def _weight(w, book, dq):
    """The weight on the GPU (q4_quantize at blocksize 64, then nf4_double_quant when dq) and the
    oracle's dequantised bf16 weight of the same inputs."""
    import torch
    import bit_nf4_quantised_amd as q
    bid, codebook = BOOKS[book]
    codes = codebook().astype(np.float64)
    qw = q.quantize_weight(to_dev(w.astype(np.float32)), double_quant=dq, codebook=bid)
    torch.cuda.synchronize()
    packed, absmax = oracle.quantize_with(w, codes, 64)
    assert np.array_equal(qw.packed.cpu().numpy(), packed)
    scales = absmax
    if dq:
        sq, c2 = oracle.double_quant(absmax)
        scales = oracle.dequant_scales(sq, c2)
    wt = oracle.dequant_blocks(packed, scales, codes, 64, w.size).reshape(w.shape)
    return qw, wt


CASES = [
    (300, 400, 960, 16, 2.0),      # fused GEMMs, ragged tiles, contraction split in two
    (513, 128, 128, 64, 0.25),     # three row tiles, the last with one row
    (40, 256, 512, 32, 1.0),       # 17..64 tokens: the small-M tile
    (3, 1040, 1088, 128, 0.5),     # few-token forward, M <= 4
    (1, 96, 4160, 32, 1.0),        #   65 blocks per row
    (16, 416, 1024, 16, 2.0),      # few-token forward at M = 16 (double-quantised scales)
]


@pytest.mark.parametrize("book", sorted(BOOKS))
@pytest.mark.parametrize("dq", [True, False], ids=["dq", "fp32scales"])
@pytest.mark.parametrize("M,N,K,r,s", CASES)
def test_codebook_weight_matches_oracle(book, dq, M, N, K, r, s):
    w, x, a, b, dy = _inputs(M + N + r, M, N, K, r)
    log(f"[codebook] {book} dq={dq} M={M} N={N} K={K} r={r}")
    qw, wt = _weight(w, book, dq)
    assert np.array_equal(gpu_dequant(qw).reshape(N, K), wt)
    y, u, dx, dA, dB = gpu_fwd_bwd(qw, x, a, b, dy, s)
    yr, ur = oracle.linear_fwd(x, wt, a, b, s)
    dxr, dar, dbr = oracle.linear_bwd(x, dy, wt, a, b, s)
    assert_close("y", f64_from_bits(y), yr)
    assert_close("u", u, ur)
    assert_close("dx", f64_from_bits(dx), dxr)
    assert_close("dA", dA, dar)
    assert_close("dB", dB, dbr)


@pytest.mark.parametrize("book", sorted(BOOKS))
@pytest.mark.parametrize("M", [1, 3, 16, 200])
def test_codebook_one_hot_rows_are_exact(book, M):
    import torch
    import bit_nf4_quantised_amd as q
    N, K, r = 384, 960, 16
    w, _, a, b, _ = _inputs(7, M, N, K, r)
    qw, wt = _weight(w, book, True)
    x = np.zeros((M, K), np.uint16)
    dy = np.zeros((M, N), np.uint16)
    for i in range(M):
        x[i, (7 * i + 3) % K] = 0x3F80
        dy[i, (5 * i + 1) % N] = 0x3F80
    y, u, dx, dA, dB = gpu_fwd_bwd(qw, x, a, np.zeros_like(b), dy, 2.0)
    for i in range(M):
        assert np.array_equal(y[i], wt[:, (7 * i + 3) % K]), i
        assert np.array_equal(dx[i], wt[(5 * i + 1) % N]), i
    # the recompute forward with the saved u equals the forward bit for bit
    X, A, B = bf16_to_dev(x), bf16_to_dev(a), bf16_to_dev(b)
    U = torch.empty(M, r, dtype=torch.float32, device=dev())
    y1 = torch.empty(M, N, dtype=torch.int16, device=dev())
    y2 = torch.empty(M, N, dtype=torch.int16, device=dev())
    ws = q.workspace(M, N, K, r)
    q.qlora_linear_fwd(qw, X, A, B, 2.0, y1, U, ws=ws)
    q.qlora_linear_fwd_recompute(qw, X, A, B, 2.0, U, y2, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits_from_dev(y1), bits_from_dev(y2))


@pytest.mark.parametrize("book", sorted(BOOKS))
@pytest.mark.parametrize("n,k,r,s", [(400, 960, 16, 2.0), (256, 1088, 64, 0.25)])
def test_codebook_merge_is_exact(book, n, k, r, s):
    import torch
    import bit_nf4_quantised_amd as q
    w, _, a, b, _ = _inputs(11 + r, 1, n, k, r)
    log(f"[codebook] merge {book} {n}x{k} r={r}")
    qw, wt = _weight(w, book, True)
    out = torch.empty(n * k, dtype=torch.int16, device=dev())
    q.qlora_merge(qw, bf16_to_dev(a), bf16_to_dev(b), s, out)
    torch.cuda.synchronize()
    got = bits_from_dev(out).reshape(n, k)
    ref = oracle.merge(wt, a, b, s)
    assert np.array_equal(got, ref), int((got != ref).sum())
