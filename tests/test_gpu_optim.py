"""GPU parity of the adapter update ("QLoRA, explained", The algorithm, step by step / Minimal
implementation): global gradient-norm clipping, then AdamW with 32-bit state over A and B.

Each step feeds the GPU's own fp32 state (p, m, v) and the same fp32 gradients to the float64
oracle, so rounding does not compound across steps, and the hyper-parameters the oracle receives
are the float32 values the C ABI passes. Bar, derived from the arithmetic (u = 2^-24, one fp32
rounding): the GPU forms each of m, v and p from at most six rounded operations on exact inputs.
v is a sum of non-negative terms, so its error is relative: |dv| <= 8u v. m can cancel, so its
error is bounded by the magnitudes that enter it: |dm| <= 8u (beta1 |m0| + (1 - beta1) c |g|).
The step divides by sqrt(v)/sqrt(1 - beta2^t) + eps (positive terms, a relative error) and
subtracts from the decayed weight: |dp| <= 16u (|p0| (1 - lr wd) + lr/(1 - beta1^t) mag_m / denom).
The norm is a double sum of exact squares (relative 1e-12), and the bf16 copy must equal torch's
round-to-nearest-even of the GPU's fp32 weights. Every call goes through one plan
(qlora_adamw_plan_*), which covers any number of tensors.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import dev, log, to_dev

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _f32(x):
    return float(np.float32(x))


def _cfgs(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_grad_norm=0.3):
    """(library config, the oracle's config holding the same float32 values)."""
    import bit_nf4_quantised_amd as q
    vals = dict(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay,
                max_grad_norm=max_grad_norm)
    return q.AdamWConfig(**vals), oracle.AdamWConfig(**{k: _f32(v) for k, v in vals.items()})


class _State:
    def __init__(self, masters, cfg, with_bf16=True, bf16_none=()):
        import torch
        import bit_nf4_quantised_amd as q
        self.p = [to_dev(x) for x in masters]
        self.m = [torch.zeros_like(x) for x in self.p]
        self.v = [torch.zeros_like(x) for x in self.p]
        self.g = [torch.empty_like(x) for x in self.p]
        self.pb = None
        if with_bf16:
            self.pb = [None if i in bf16_none else
                       torch.full((x.numel(),), 0x7fc1, dtype=torch.int16, device=dev())
                       for i, x in enumerate(self.p)]
        self.norm = torch.full((1,), -1.0, dtype=torch.float64, device=dev())
        self.plan = q.AdamWPlan(self.p, self.g, self.m, self.v, self.pb, cfg)

    def host(self):
        f = lambda ts: [t.cpu().numpy().astype(np.float64) for t in ts]  # noqa: E731
        return f(self.p), f(self.m), f(self.v)


def _step_gpu(st, grads, step):
    import torch
    for t, g in zip(st.g, grads):
        t.copy_(torch.from_numpy(g).reshape(t.shape))
    st.plan.step(step, st.norm)
    torch.cuda.synchronize()


def _check_step(name, prev, grads, got, ref, ocfg, step, norm):
    p0, m0, v0 = prev
    pg, mg, vg = got
    pr, mr, vr, _ = ref
    c = oracle.clip_coefficient(norm, ocfg.max_grad_norm)
    b1, b2 = ocfg.beta1, ocfg.beta2
    step_size = ocfg.lr / (1.0 - b1 ** step)
    decay = 1.0 - ocfg.lr * ocfg.weight_decay
    worst = [0.0, 0.0, 0.0]
    for i in range(len(p0)):
        mag_m = b1 * np.abs(m0[i]) + (1.0 - b1) * c * np.abs(grads[i].astype(np.float64))
        denom = np.sqrt(vr[i] / (1.0 - b2 ** step)) + ocfg.eps
        bm = 8 * U * mag_m
        bv = 8 * U * vr[i]
        bp = 16 * U * (np.abs(p0[i]) * decay + step_size * mag_m / denom)
        for j, (d, b, what) in enumerate(((np.abs(mg[i] - mr[i]), bm, "m"), (np.abs(vg[i] - vr[i]), bv, "v"),
                                          (np.abs(pg[i] - pr[i]), bp, "p"))):
            bad = d > b
            assert not bad.any(), (f"{name} step {step} tensor {i}: {int(bad.sum())} {what} values "
                                   f"outside the bound, worst {float((d - b).max()):.3e}")
            worst[j] = max(worst[j], float(np.max(d / np.maximum(b, 1e-300))))
    log(f"[optim] {name} step {step}: norm {norm:.5f} clip {c:.5f}; worst error / bound "
        f"m {worst[0]:.3f} v {worst[1]:.3f} p {worst[2]:.3f}")


def _run(name, shapes, cfg_kw, steps, sigma, with_bf16=True, workload="llama8b"):
    import torch
    cfg, ocfg = _cfgs(**cfg_kw)
    st = _State(wl.adapter_masters(workload, shapes), cfg, with_bf16)
    for step in range(1, steps + 1):
        grads = wl.adapter_grads(workload, shapes, step, sigma)
        prev = st.host()
        _step_gpu(st, grads, step)
        g64 = [g.astype(np.float64) for g in grads]
        ref = oracle.adamw_step(prev[0], g64, prev[1], prev[2], step, ocfg)
        sq_ref = sum(float(np.sum(g * g)) for g in g64)
        assert ref[3] == pytest.approx(np.sqrt(sq_ref), rel=1e-15)
        assert float(st.norm.cpu()[0]) == pytest.approx(ref[3], rel=1e-12)
        got = st.host()
        _check_step(name, prev, grads, got, ref, ocfg, step, ref[3])
        if st.pb is not None:
            for i, (p, pb) in enumerate(zip(st.p, st.pb)):
                want = p.cpu().to(torch.bfloat16).view(torch.int16).reshape(-1)
                assert torch.equal(pb.cpu(), want), f"{name}: bf16 copy of tensor {i} differs"
    return st


@pytest.mark.parametrize("max_norm,sigma", [(0.3, 1e-3), (0.3, 1e-5), (0.0, 1e-3)],
                         ids=["clipped", "below-threshold", "no-clipping"])
def test_llama8b_layer_adapters(max_norm, sigma):
    # the 14 adapter tensors of one Llama-3.1-8B layer at rank 16 (1.31 M values), three steps
    shapes = wl.adapter_shapes(wl.WORKLOADS["llama8b"])
    log(f"[optim] llama8b layer: {len(shapes)} tensors, max_norm {max_norm}, grad sigma {sigma}")
    _run(f"llama8b-layer {max_norm}/{sigma}", shapes, dict(max_grad_norm=max_norm), 3, sigma)


def test_llama70b_layer_rank64():
    shapes = wl.adapter_shapes(wl.WORKLOADS["llama70b"])
    log(f"[optim] llama70b layer, rank 64: {len(shapes)} tensors")
    _run("llama70b-layer", shapes, dict(lr=1e-4, weight_decay=0.0), 2, 2e-4, workload="llama70b")


def test_ragged_and_tiny_tensors():
    # sizes that end inside a 4096-value chunk and inside a float4, and a chunk count that leaves the
    # last norm group of four partly empty (1 + 6 + 2 + 1 + 1 + 1 + 3 + 1 chunks per pattern, x 5
    # = 80, plus 3 single-chunk tensors: 83 chunks in 21 groups); no bf16 copies
    shapes = [(16, 40), (24, 1024), (4100, 1), (1, 4), (3, 4), (4096, 1), (8196, 1), (16, 8)] * 5 + \
        [(4, 1)] * 3
    log(f"[optim] ragged: {len(shapes)} tensors")
    _run("ragged", shapes, dict(lr=3e-3, weight_decay=0.05), 4, 0.05, with_bf16=False)


def test_zero_gradient_and_large_step():
    import torch
    shapes = [(16, 4096), (4096, 16)]
    cfg, ocfg = _cfgs(lr=1e-3, weight_decay=0.1)
    st = _State(wl.adapter_masters("llama8b", shapes), cfg, bf16_none=(1,))
    p0 = st.host()
    zeros = [np.zeros(s, dtype=np.float32) for s in shapes]
    _step_gpu(st, zeros, 1000)
    assert float(st.norm.cpu()[0]) == 0.0
    got = st.host()
    ref = oracle.adamw_step(p0[0], [z.astype(np.float64) for z in zeros], p0[1], p0[2], 1000, ocfg)
    _check_step("zero-grad", p0, zeros, got, ref, ocfg, 1000, 0.0)
    assert all(np.all(x == 0) for x in got[1] + got[2])
    assert torch.equal(st.pb[0].cpu(), st.p[0].cpu().to(torch.bfloat16).view(torch.int16).reshape(-1))


def test_norm_is_reproducible_and_scales_exactly():
    # the same gradients give the same norm bit for bit; doubling every gradient (exact in fp32)
    # doubles the norm exactly (sqrt(4 s) = 2 sqrt(s) in IEEE arithmetic)
    shapes = wl.adapter_shapes(wl.WORKLOADS["llama8b"])
    cfg, _ = _cfgs()
    st = _State(wl.adapter_masters("llama8b", shapes), cfg)
    grads = wl.adapter_grads("llama8b", shapes, 9)
    _step_gpu(st, grads, 1)
    first = float(st.norm.cpu()[0])
    _step_gpu(st, grads, 2)
    assert float(st.norm.cpu()[0]) == first
    _step_gpu(st, [2 * g for g in grads], 3)
    assert float(st.norm.cpu()[0]) == 2 * first
    ref = np.sqrt(sum(float(np.sum(g.astype(np.float64) ** 2)) for g in grads))
    assert first == pytest.approx(ref, rel=1e-12)


def test_full_model_adapters_one_step():
    # the launch configuration the benchmark times: every adapter of a 32-layer Llama-3.1-8B at
    # rank 16 (448 tensors, 41.9 M values) in one plan, one step, every value against the oracle
    shapes = wl.adapter_shapes(wl.WORKLOADS["llama8b"], wl.LLAMA8B_LAYERS)
    log(f"[optim] full model: {len(shapes)} tensors")
    _run("llama8b-model", shapes, {}, 1, 1e-3)
