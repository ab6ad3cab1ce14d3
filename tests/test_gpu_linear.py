"""GPU parity of the adapted linear's forward and backward against the oracle.

Tolerance (bf16 inputs, fp32 accumulation): relative Frobenius error <= 5e-3 and elementwise
|err| <= 1e-2 * max|ref|, for y, dX, dA and dB separately; u = x A^T is checked the same way.
Exact special cases pin layout and transposition: with B = 0, one-hot rows of x give rows of y that
equal columns of the dequantised weight bit for bit, and one-hot rows of dY give rows of dX equal
to rows of it.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import (assert_close, f64_from_bits, gpu_fwd_bwd, gpu_quantize, log,
                         oracle_weight)

pytestmark = pytest.mark.gpu


def _inputs(seed, M, N, K, r, kind="gauss", sigma=0.02):
    w = wl.weight("single", 200 + seed, N, K, kind, sigma)
    g = wl.rng_for("single", 200 + seed, "x")
    x = wl.to_bf16_bits(g.standard_normal((M, K), dtype=np.float32))
    a = wl.to_bf16_bits(g.standard_normal((r, K), dtype=np.float32) * np.float32(0.01))
    b = wl.to_bf16_bits(g.standard_normal((N, r), dtype=np.float32) * np.float32(0.01))
    dy = wl.to_bf16_bits(g.standard_normal((M, N), dtype=np.float32))
    return w, x, a, b, dy


def check_full(w, x, a, b, dy, s, name, accumulate=False, dA0=None, dB0=None):
    N, K = w.shape
    M = x.shape[0]
    log(f"[linear] {name} M={M} N={N} K={K} r={a.shape[0]} s={s}")
    qw = gpu_quantize(w)[0]
    y, u, dx, dA, dB = gpu_fwd_bwd(qw, x, a, b, dy, s, accumulate=accumulate, dA0=dA0, dB0=dB0)
    wt = oracle_weight(w)
    yr, ur = oracle.linear_fwd(x, wt, a, b, s)
    dxr, dar, dbr = oracle.linear_bwd(x, dy, wt, a, b, s)
    if accumulate:
        dar = dar + dA0
        dbr = dbr + dB0
    assert_close("y", f64_from_bits(y), yr)
    assert_close("u", u, ur)
    assert_close("dx", f64_from_bits(dx), dxr)
    assert_close("dA", dA, dar)
    assert_close("dB", dB, dbr)
    return y, u, dx, dA, dB


def test_single_linear_workload():
    wlk = wl.WORKLOADS["single"]
    w, x, a, b, dy = wl.linear_inputs(wlk, 0, wlk.linears[0])
    check_full(w, x, a, b, dy, wlk.scale, "single")


@pytest.mark.parametrize("M,N,K,r,s", [
    (300, 400, 960, 16, 2.0),      # ragged in every tile dimension
    (300, 400, 960, 64, 0.25),
    (77, 1040, 1088, 128, 0.5),    # one partial row tile, rank 128
    (40, 256, 512, 32, 1.0),       # 17..64 tokens: small-M tile
    (16, 4096, 4096, 16, 2.0),     # 16 tokens on a 4096x4096 weight: dX in 8 contraction ranges
    (40, 1040, 2112, 16, 0.5),     #   two ranges, the second ending in a partial step
    (100, 2048, 1024, 32, 1.0),    #   128-row dX tiles in 4 ranges
    (40, 4096, 2048, 16, 2.0),     # 17..64 tokens: the forward in 4 contraction ranges, dX in 8
    (64, 2064, 4160, 16, 0.5),     #   forward in 8 ranges, the last of 2 steps; dX in 2, ragged
    (513, 128, 128, 16, 2.0),      # three row tiles, the last with one row
    (1, 400, 960, 16, 2.0),        # skinny forward
    (4, 400, 960, 64, 0.25),
    (16, 416, 1024, 16, 2.0),
    (16, 64, 64, 16, 2.0),         # one block per row
    (2, 400, 960, 16, 2.0),        # M <= 4: four rows x four chunks per MFMA
    (3, 1040, 1088, 128, 0.5),     #   rank 128, ragged rows
    (1, 64, 64, 16, 2.0),          #   one block per row
    (4, 96, 4160, 32, 1.0),        #   65 blocks per row: a 64-column last step, odd scale offsets
    (1, 16, 2048, 64, 1.0),        #   fewer rows than one row block; the adapter needs four blocks
    (4, 208, 16448, 16, 2.0),      #   257 blocks per row: groups of 256 blocks split steps
    (1800, 14336, 128, 16, 2.0),   # forward: 896 tiles of 256 rows, ragged last row block
    (1800, 128, 14336, 16, 2.0),   # the same for the dX GEMM (14336 output columns)
    (1500, 1040, 2112, 16, 2.0),   # 256-row tiles with the contraction in 4 ranges (54 tiles, the
    (1536, 1024, 2048, 64, 0.5),   #   last range shorter), ragged rows and columns; then exact fit
    (300, 16512, 2048, 16, 2.0),   # forward: 258 tiles of 256 rows, the 2 past the first round of 256
                                   #   CUs in 4 contraction ranges each (the tail), ragged rows
    (300, 2048, 16512, 16, 2.0),   # the same for the dX GEMM (16512 output columns)
    # ranks that are not a power of two: the adapter kernels, the fused GEMMs' partial adapter steps
    # (r > 64: two steps, the second partial) and the few-token epilogue's u runs (256 / r rounds down)
    (300, 400, 960, 48, 1.0),      #   GEMM with a split contraction
    (700, 1040, 4160, 48, 0.5),    #   rank-48 adapter passes: three row blocks, ragged column ranges
    (300, 400, 960, 80, 0.5),
    (300, 400, 960, 96, 0.5),
    (300, 400, 960, 112, 0.25),
    (3, 400, 960, 48, 1.0),        #   M <= 4 few-token kernel
    (1, 1040, 1088, 112, 0.25),
    (16, 416, 1024, 80, 0.5),      #   16-row few-token kernel
    (16, 416, 1024, 112, 0.25),
])
def test_ragged_shapes(M, N, K, r, s):
    check_full(*_inputs(M * 7 + r, M, N, K, r), s, "ragged")


def test_accumulate_mode():
    M, N, K, r = 96, 256, 512, 16
    w, x, a, b, dy = _inputs(9, M, N, K, r)
    rng = np.random.default_rng(9)
    dA0 = rng.standard_normal((r, K)).astype(np.float32)
    dB0 = rng.standard_normal((N, r)).astype(np.float32)
    check_full(w, x, a, b, dy, 2.0, "accumulate", accumulate=True, dA0=dA0, dB0=dB0)


@pytest.mark.parametrize("M", [1, 3, 8, 200])
def test_one_hot_rows_are_exact(M):
    """B = 0 and one-hot rows: y rows are columns of W~ and dX rows are rows of W~, bit for bit."""
    N, K, r = 256, 512, 16
    w, x, a, b, dy = _inputs(13, M, N, K, r)
    b = np.zeros_like(b)
    x = np.zeros_like(x)
    cols = (np.arange(M) * 37) % K
    x[np.arange(M), cols] = 0x3F80                      # bf16 1.0
    dy = np.zeros_like(dy)
    rows = (np.arange(M) * 11) % N
    dy[np.arange(M), rows] = 0x3F80
    log(f"[linear] one-hot M={M}")
    qw = gpu_quantize(w)[0]
    y, u, dx, dA, dB = gpu_fwd_bwd(qw, x, a, b, dy, 2.0)
    wt = oracle_weight(w)
    assert np.array_equal(y, wt[:, cols].T), "y rows must equal columns of W~"
    assert np.array_equal(dx, wt[rows, :]), "dX rows must equal rows of W~"


def test_zero_weight_gives_adapter_term():
    M, N, K, r = 64, 256, 512, 16
    w, x, a, b, dy = _inputs(14, M, N, K, r)
    check_full(np.zeros_like(w), x, a, b, dy, 2.0, "zero weight")


def test_zero_input():
    M, N, K, r = 64, 256, 512, 16
    w, x, a, b, dy = _inputs(15, M, N, K, r)
    x = np.zeros_like(x)
    log("[linear] zero x")
    qw = gpu_quantize(w)[0]
    y, u, dx, dA, dB = gpu_fwd_bwd(qw, x, a, b, dy, 2.0)
    assert not f64_from_bits(y).any() and not u.any() and not dA.any() and not dB.any()


def test_fwd_bwd_deterministic():
    M, N, K, r = 300, 400, 960, 16
    w, x, a, b, dy = _inputs(16, M, N, K, r)
    log("[linear] determinism")
    qw = gpu_quantize(w)[0]
    r1 = gpu_fwd_bwd(qw, x, a, b, dy, 2.0)
    r2 = gpu_fwd_bwd(qw, x, a, b, dy, 2.0)
    for p, q_ in zip(r1, r2):
        assert np.array_equal(p, q_)


@pytest.mark.parametrize("M", [8, 300])
def test_forward_recompute_matches_forward(M):
    """The recompute entry (u given) reproduces the forward's y bit for bit."""
    import torch
    import bit_nf4_quantised_amd as q
    from gpu_helpers import bf16_to_dev, dev
    N, K, r = 400, 960, 16
    w, x, a, b, dy = _inputs(17 + M, M, N, K, r)
    log(f"[linear] recompute M={M}")
    qw = gpu_quantize(w)[0]
    X, A, B = bf16_to_dev(x), bf16_to_dev(a), bf16_to_dev(b)
    y1 = torch.empty(M, N, dtype=torch.int16, device=dev())
    y2 = torch.empty(M, N, dtype=torch.int16, device=dev())
    u = torch.empty(M, r, dtype=torch.float32, device=dev())
    q.qlora_linear_fwd(qw, X, A, B, 2.0, y1, u)
    q.qlora_linear_fwd_recompute(qw, X, A, B, 2.0, u, y2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


# ---------------------------------------------------------------- fp32 scales (no double quantisation)
def _f32s_weight(w):
    import bit_nf4_quantised_amd as q
    from gpu_helpers import to_dev
    import torch
    qw = q.quantize_weight(to_dev(w.astype(np.float32)), double_quant=False)
    torch.cuda.synchronize()
    packed, absmax = oracle.quantize(w)
    wt = oracle.dequant_blocks(packed, absmax, oracle.codebook(), 64, w.size).reshape(w.shape)
    return qw, wt


@pytest.mark.parametrize("M,N,K,r,s", [
    (300, 400, 960, 16, 2.0),      # ragged in every tile dimension, K % 128 == 64
    (513, 128, 128, 64, 0.25),     # three row tiles, the last with one row
    (77, 1040, 1088, 128, 0.5),
    (8, 400, 960, 16, 2.0),        # 5..16 tokens: the 16-row few-token kernel with fp32 scales
    (16, 4096, 512, 16, 2.0),      #   one 512-column step per row block
    (5, 1040, 4160, 128, 0.5),     #   65 blocks per row (a 64-column last step), ragged rows
    (13, 528, 2112, 48, 1.0),      #   rank 48, a row block of 16 rows past its last whole tile
    (1, 400, 960, 16, 2.0),        # M <= 4: the few-token kernel with fp32 scales
    (4, 96, 4160, 32, 1.0),        #   65 blocks per row, a 64-column last step
    (3, 1040, 1088, 128, 0.5),     #   rank 128, ragged rows
    (2048, 4096, 4096, 16, 2.0),   # the q/o shape of the 8B layer set
    (1500, 1040, 2112, 16, 2.0),   # 256-row tiles, contraction in 4 ranges
])
def test_fp32_scale_weight_matches_oracle(M, N, K, r, s):
    from gpu_helpers import gpu_dequant
    w, x, a, b, dy = _inputs(M + N + r, M, N, K, r)
    log(f"[linear] fp32 scales M={M} N={N} K={K} r={r}")
    qw, wt = _f32s_weight(w)
    assert np.array_equal(gpu_dequant(qw).reshape(N, K), wt)
    y, u, dx, dA, dB = gpu_fwd_bwd(qw, x, a, b, dy, s)
    yr, ur = oracle.linear_fwd(x, wt, a, b, s)
    dxr, dar, dbr = oracle.linear_bwd(x, dy, wt, a, b, s)
    assert_close("y", f64_from_bits(y), yr)
    assert_close("dx", f64_from_bits(dx), dxr)
    assert_close("dA", dA, dar)
    assert_close("dB", dB, dbr)


@pytest.mark.parametrize("M", [3, 9, 200])
def test_fp32_scale_weight_one_hot_and_recompute(M):
    # with B = 0, one-hot rows of x give y rows equal to columns of W~ bit for bit, one-hot rows of
    # dY give dX rows equal to rows of W~; the recompute forward equals the forward (M = 3: the
    # four-row few-token kernel, M = 9: the 16-row one, M = 200: the fused GEMM)
    import torch
    import bit_nf4_quantised_amd as q
    from gpu_helpers import bf16_to_dev, bits_from_dev, dev
    N, K, r = 384, 960, 16
    w, x, a, b, dy = _inputs(5, M, N, K, r)
    qw, wt = _f32s_weight(w)
    x = np.zeros((M, K), np.uint16)
    dy = np.zeros((M, N), np.uint16)
    for i in range(M):
        x[i, (7 * i) % K] = 0x3F80
        dy[i, (5 * i) % N] = 0x3F80
    b0 = np.zeros_like(b)
    y, u, dx, dA, dB = gpu_fwd_bwd(qw, x, a, b0, dy, 2.0)
    for i in range(M):
        assert np.array_equal(y[i], wt[:, (7 * i) % K]), i
        assert np.array_equal(dx[i], wt[(5 * i) % N]), i
    X, A, B = bf16_to_dev(x), bf16_to_dev(a), bf16_to_dev(b)
    U = torch.empty(M, r, dtype=torch.float32, device=dev())
    y1 = torch.empty(M, N, dtype=torch.int16, device=dev())
    y2 = torch.empty(M, N, dtype=torch.int16, device=dev())
    q.qlora_linear_fwd(qw, X, A, B, 2.0, y1, U)
    q.qlora_linear_fwd_recompute(qw, X, A, B, 2.0, U, y2)
    torch.cuda.synchronize()
    assert np.array_equal(bits_from_dev(y1), bits_from_dev(y2))
    with pytest.raises(q.NF4Error):
        q.qlora_merge(qw, A, B, 2.0, torch.empty(N * K, dtype=torch.int16, device=dev()))
