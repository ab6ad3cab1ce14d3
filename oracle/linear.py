"""The adapted linear layer's forward and backward in float64. TEST INFRASTRUCTURE ONLY.

Inputs are bf16 bit patterns (uint16 arrays) so that the oracle and the GPU path consume identical
values; each is widened exactly to float64 and the products are plain float64 matrix products.
"""
from __future__ import annotations

import numpy as np


def _f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def linear_fwd(x_bits, w_bits, a_bits, b_bits, scale: float):
    """Forward of an adapted linear: y = X W~^T + s (X A^T) B^T; also returns u = X A^T.

    "QLoRA, explained", The forward pass and gradients (its display equation was lost) and
    The algorithm, step by step (the forward line of its pseudo-code): the frozen dequantised
    weight's product plus the adapter product scaled by s = lora_alpha / r. No bias and no dropout.

    Shapes: X [M, K], W~ [N, K] (the dequantised bf16 weight), A [r, K], B [N, r].
    Returns (y [M, N], u [M, r]) in float64.
    """
    return linear_fwd_f64(_f64(x_bits), _f64(w_bits), _f64(a_bits), _f64(b_bits), scale)


def linear_fwd_f64(x, w, a, b, scale: float):
    """``linear_fwd`` on float64 arrays (same formula; used by the finite-difference pins)."""
    u = x @ a.T
    y = x @ w.T + scale * (u @ b.T)
    return y, u


def linear_bwd(x_bits, dy_bits, w_bits, a_bits, b_bits, scale: float):
    """Backward of an adapted linear given the upstream gradient dY (the pages' delta).

    "QLoRA, explained", The forward pass and gradients: the adapter gradients are LoRA's with W~ in
    place of W0, dL/dB = gamma G A^T and dL/dA = gamma B^T G, and the input gradient is
    dL/dX = delta (W~ + gamma B A); W~ itself gets no gradient. G, not defined on the page, is read
    as the gradient with respect to the whole weight, G = delta^T X.

    Shapes: X [M, K], dY [M, N], W~ [N, K], A [r, K], B [N, r].
    Returns (dX [M, K], dA [r, K], dB [N, r]) in float64.
    """
    return linear_bwd_f64(_f64(x_bits), _f64(dy_bits), _f64(w_bits), _f64(a_bits), _f64(b_bits),
                          scale)


def linear_bwd_f64(x, dy, w, a, b, scale: float):
    """``linear_bwd`` on float64 arrays (same formulas)."""
    g = dy.T @ x
    d_b = scale * (g @ a.T)
    d_a = scale * (b.T @ g)
    d_x = dy @ (w + scale * (b @ a))
    return d_x, d_a, d_b


def linear_bwd_sampled(x_bits, dy_bits, w_bits, a_bits, b_bits, scale: float, x_rows, a_cols, b_rows):
    """``linear_bwd`` restricted to a sample of outputs, for sizes where G = dY^T X (N x K) is too
    large to form: rows ``x_rows`` of dX, columns ``a_cols`` of dA and rows ``b_rows`` of dB.

    Same formulas, restricted: dX[i] = dY[i] (W~ + s B A); dA[:, c] = s B^T G[:, c] with
    G[:, c] = dY^T X[:, c]; dB[n] = s G[n] A^T with G[n] = dY[:, n]^T X.
    """
    x, dy, w, a, b = _f64(x_bits), _f64(dy_bits), _f64(w_bits), _f64(a_bits), _f64(b_bits)
    x_rows, a_cols, b_rows = np.asarray(x_rows), np.asarray(a_cols), np.asarray(b_rows)
    d_x = dy[x_rows] @ (w + scale * (b @ a))
    g_cols = dy.T @ x[:, a_cols]
    d_a = scale * (b.T @ g_cols)
    g_rows = dy[:, b_rows].T @ x
    d_b = scale * (g_rows @ a.T)
    return d_x, d_a, d_b
