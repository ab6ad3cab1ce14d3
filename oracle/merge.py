"""The adapter merged into the dequantised base weight, in bf16. TEST INFRASTRUCTURE ONLY.

"QLoRA, explained", Quality loss at merge time: training saw W~, the dequantised weight, never the
original one, so the merge that preserves the trained model adds the adapter to W~ and serves the
sum in bf16. The pages fix no arithmetic for the sum; the reading taken is
the plainest one: the exact value W~ + s B A (s = lora_alpha / r, as in the forward), rounded once
to bf16 (round to nearest, ties to even). Here the sum is formed in float64 from the exact bf16
values of W~, A and B, whose error is far below half a bf16 unit.
"""
from __future__ import annotations

import numpy as np


def _f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_bits_from_f64(x) -> np.ndarray:
    """Round float64 values to bfloat16 in one step (round to nearest, ties to even), without
    passing through float32. The value is split as m * 2^e with 0.5 <= |m| < 1; bf16 keeps 8
    significant bits, so m * 2^8 is rounded to an integer (exact float64 arithmetic, rint rounds
    ties to even). Zero and normal bf16 results only: magnitudes below 2^-126 are rejected."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value")
    if np.any((x != 0) & (np.abs(x) < 2.0 ** -126)):
        raise ValueError("bf16 subnormal range not supported")
    m, e = np.frexp(x)
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)      # exactly representable in bf16
    u = r.astype(np.float32).view(np.uint32)          # exact: 8 significant bits
    return (u >> 16).astype(np.uint16)


def merge(w_bits, a_bits, b_bits, scale: float) -> np.ndarray:
    """bf16(W~ + s B A) as bf16 bit patterns [N, K].

    Shapes: W~ [N, K] (the dequantised weight, bf16 bits), A [r, K], B [N, r] (bf16 bits)."""
    w = _f64(w_bits)
    v = w + scale * (_f64(b_bits) @ _f64(a_bits))
    return bf16_bits_from_f64(v).reshape(w.shape)
