"""The pages' numpy toy run: relative quantisation error of 4-bit codebooks and how much of the
quantisation residual a low-rank term captures. TEST INFRASTRUCTURE ONLY; these functions exist to
pin the oracle's quantiser to the numbers the page prints.

"QLoRA, explained", A toy run: how much does NF4 lose, and can LoRA win it back?
"""
from __future__ import annotations

import numpy as np

from .nf4 import codebook, quantize_blocks


def int4_codebook() -> np.ndarray:
    """The toy's symmetric 15-level INT4 grid in [-1, 1]: k / 7 for k = -7..7."""
    return (np.arange(-7, 8, dtype=np.float64) / 7.0).astype(np.float32)


def fp4_codebook() -> np.ndarray:
    """The toy's FP4 codebook, E2M1 rescaled into [-1, 1]: magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} / 6 with
    both signs (the two zeros coincide), 15 distinct values."""
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]) / 6.0
    vals = np.unique(np.concatenate([-mags, mags]))
    return vals.astype(np.float32)


def _reconstruct(w, codes, blocksize):
    idx, absmax = quantize_blocks(w, blocksize, codes)
    return codes.astype(np.float64)[idx] * absmax.astype(np.float64)[:, None]


def relative_mse(w, codes=None, blocksize: int = 64) -> float:
    """E[(w~ - w)^2] / E[w^2] for blockwise absmax quantisation with the given codebook (no double
    quantisation, reconstruction in float64), as the toy run reports it."""
    codes = codebook() if codes is None else np.asarray(codes, dtype=np.float32)
    w = np.asarray(w, dtype=np.float64).reshape(-1)
    rec = _reconstruct(w.astype(np.float32), codes, blocksize).reshape(-1)
    w32 = w.astype(np.float32).astype(np.float64)
    return float(np.mean((rec - w32) ** 2) / np.mean(w32 ** 2))


def residual_capture(w2d, ranks, codes=None, blocksize: int = 64):
    """Share of the residual energy ||W - W~||^2 held by its best rank-k approximation, for each k.

    The best rank-k approximation keeps the k largest singular values (Eckart-Young), so the share is
    sum of the k largest squared singular values over the sum of all of them."""
    codes = codebook() if codes is None else np.asarray(codes, dtype=np.float32)
    w2d = np.asarray(w2d, dtype=np.float32)
    rec = _reconstruct(w2d, codes, blocksize).reshape(w2d.shape)
    s = np.linalg.svd(w2d.astype(np.float64) - rec, compute_uv=False)
    e = s ** 2
    return [float(e[:k].sum() / e.sum()) for k in ranks]
