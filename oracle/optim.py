"""The adapter update of a training step: gradient-norm clipping, then AdamW. TEST INFRASTRUCTURE ONLY.

"QLoRA, explained", The algorithm, step by step: once the backward pass has produced them, the
gradients of A and B are clipped by their global norm (0.3 in the original runs) and an AdamW optimiser (32-bit state, or 8-bit,
optionally paged) updates A and B only; "Minimal implementation" shows torch's AdamW with lr 2e-4
and clip_grad_norm_(..., 0.3). The pages fix no other constants, so the reading taken is the
plainest one: the AdamW of Loshchilov and Hutter with decoupled weight decay, in the form torch
documents, with torch's defaults for what the pages leave open (beta1 0.9, beta2 0.999, eps 1e-8,
weight decay 0.01) and torch's clipping rule (coefficient max_norm / (norm + 1e-6), never above 1).
32-bit state: master weights, first and second moments in fp32 on the GPU; here every quantity is
float64.

For parameter p with gradient g at step t (t = 1, 2, ...), after clipping g <- c g:
    p <- p (1 - lr wd)
    m <- beta1 m + (1 - beta1) g
    v <- beta2 v + (1 - beta2) g^2
    p <- p - lr (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class AdamWConfig:
    lr: float = 2e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    max_grad_norm: float = 0.3     # <= 0: no clipping


def global_grad_norm(grads) -> float:
    """L2 norm over every element of every gradient tensor."""
    return float(np.sqrt(sum(float(np.sum(np.asarray(g, dtype=np.float64) ** 2)) for g in grads)))


def clip_coefficient(norm: float, max_norm: float) -> float:
    """Factor the gradients are multiplied by: max_norm / (norm + 1e-6), at most 1."""
    if max_norm <= 0:
        return 1.0
    return min(1.0, max_norm / (norm + 1e-6))


def adamw_step(params, grads, exp_avg, exp_avg_sq, step: int, cfg: AdamWConfig):
    """One clipped AdamW step over a list of tensors. Returns (params, exp_avg, exp_avg_sq, norm)
    as new float64 arrays (inputs are not modified); `norm` is the gradient norm before clipping."""
    if step < 1:
        raise ValueError("steps count from 1")
    norm = global_grad_norm(grads)
    c = clip_coefficient(norm, cfg.max_grad_norm)
    bc1 = 1.0 - cfg.beta1 ** step
    bc2 = 1.0 - cfg.beta2 ** step
    out_p, out_m, out_v = [], [], []
    for p, g, m, v in zip(params, grads, exp_avg, exp_avg_sq):
        p = np.array(p, dtype=np.float64)
        g = np.asarray(g, dtype=np.float64) * c
        m = cfg.beta1 * np.asarray(m, dtype=np.float64) + (1.0 - cfg.beta1) * g
        v = cfg.beta2 * np.asarray(v, dtype=np.float64) + (1.0 - cfg.beta2) * g * g
        p = p * (1.0 - cfg.lr * cfg.weight_decay)
        p = p - cfg.lr * (m / bc1) / (np.sqrt(v / bc2) + cfg.eps)
        out_p.append(p)
        out_m.append(m)
        out_v.append(v)
    return out_p, out_m, out_v, norm
