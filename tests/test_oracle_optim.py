"""Pins of the oracle's adapter update (gradient-norm clipping, then AdamW).

"QLoRA, explained", The algorithm, step by step / Minimal implementation: clip the adapter gradients
by their global norm (0.3), then AdamW over A and B. The oracle is pinned to torch's own float64
AdamW and clip_grad_norm_ (an independent implementation of the same published algorithm), and to
closed forms: the first step of Adam moves every element by lr * g / (|g| + eps), a zero gradient
only decays the weights, and the first moment after one step is (1 - beta1) times the clipped
gradient.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.optim import AdamWConfig


def _tensors(seed, shapes, scale=1.0):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(s) * scale for s in shapes]


SHAPES = [(16, 96), (80, 16), (16, 40), (24, 16)]


@pytest.mark.parametrize("max_norm", [0.3, 0.0, 50.0])
def test_matches_torch_adamw_with_clipping(max_norm):
    cfg = AdamWConfig(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_grad_norm=max_norm)
    p0 = _tensors(1, SHAPES, 0.02)
    tp = [torch.tensor(p, dtype=torch.float64, requires_grad=True) for p in p0]
    opt = torch.optim.AdamW(tp, lr=cfg.lr, betas=(cfg.beta1, cfg.beta2), eps=cfg.eps,
                            weight_decay=cfg.weight_decay)
    p = [x.copy() for x in p0]
    m = [np.zeros(s) for s in SHAPES]
    v = [np.zeros(s) for s in SHAPES]
    for step in range(1, 6):
        grads = _tensors(100 + step, SHAPES, 0.05 * step)
        for t, g in zip(tp, grads):
            t.grad = torch.tensor(g, dtype=torch.float64)
        tnorm = float(torch.linalg.vector_norm(torch.cat([t.grad.flatten() for t in tp])))
        if max_norm > 0:
            tnorm = float(torch.nn.utils.clip_grad_norm_(tp, max_norm))
        opt.step()
        p, m, v, norm = oracle.adamw_step(p, grads, m, v, step, cfg)
        assert norm == pytest.approx(tnorm, rel=1e-13)
        for i, t in enumerate(tp):
            st = opt.state[t]
            np.testing.assert_allclose(p[i], t.detach().numpy(), rtol=1e-12, atol=1e-17)
            np.testing.assert_allclose(m[i], st["exp_avg"].numpy(), rtol=1e-12, atol=1e-20)
            np.testing.assert_allclose(v[i], st["exp_avg_sq"].numpy(), rtol=1e-12, atol=1e-24)


def test_first_step_closed_form():
    # m/(1-beta1) = g and sqrt(v/(1-beta2)) = |g| after one step: each element moves by
    # lr * g / (|g| + eps), whatever the gradient's scale
    cfg = AdamWConfig(lr=1e-3, weight_decay=0.0, max_grad_norm=0.0)
    p0 = _tensors(3, SHAPES, 0.1)
    g = _tensors(4, SHAPES, 7.0)
    z = [np.zeros(s) for s in SHAPES]
    p1, m1, v1, _ = oracle.adamw_step(p0, g, z, z, 1, cfg)
    for a, b, gg in zip(p0, p1, g):
        np.testing.assert_allclose(a - b, cfg.lr * gg / (np.abs(gg) + cfg.eps), rtol=1e-12)


def test_zero_gradient_only_decays():
    cfg = AdamWConfig(lr=5e-3, weight_decay=0.1)
    p = _tensors(5, SHAPES, 1.0)
    start = [x.copy() for x in p]
    m = [np.zeros(s) for s in SHAPES]
    v = [np.zeros(s) for s in SHAPES]
    g = [np.zeros(s) for s in SHAPES]
    for step in range(1, 4):
        p, m, v, norm = oracle.adamw_step(p, g, m, v, step, cfg)
        assert norm == 0.0
    for a, b in zip(start, p):
        np.testing.assert_allclose(b, a * (1 - cfg.lr * cfg.weight_decay) ** 3, rtol=1e-14)
    assert all(np.all(x == 0) for x in m + v)


def test_clipping_scales_the_first_moment():
    cfg = AdamWConfig(max_grad_norm=0.3)
    g = _tensors(6, SHAPES, 1.0)
    norm = float(np.linalg.norm(np.concatenate([x.ravel() for x in g])))
    assert norm > 1.0
    c = 0.3 / (norm + 1e-6)
    z = [np.zeros(s) for s in SHAPES]
    _, m1, v1, n = oracle.adamw_step(_tensors(7, SHAPES), g, z, z, 1, cfg)
    assert n == pytest.approx(norm, rel=1e-14)
    for gg, mm, vv in zip(g, m1, v1):
        np.testing.assert_allclose(mm, (1 - cfg.beta1) * c * gg, rtol=1e-14)
        np.testing.assert_allclose(vv, (1 - cfg.beta2) * (c * gg) ** 2, rtol=1e-13)
    # below the threshold nothing is scaled
    small = [x * 1e-3 for x in g]
    _, m2, _, _ = oracle.adamw_step(_tensors(7, SHAPES), small, z, z, 1, cfg)
    for gg, mm in zip(small, m2):
        np.testing.assert_allclose(mm, (1 - cfg.beta1) * gg, rtol=1e-14)


def test_steps_count_from_one():
    with pytest.raises(ValueError):
        oracle.adamw_step([np.zeros(2)], [np.zeros(2)], [np.zeros(2)], [np.zeros(2)], 0, AdamWConfig())
