"""A training step captured in a HIP graph and replayed: every per-step call of the library is a
plain sequence of kernel launches (no allocation, copy, memset or synchronisation), so a caller can
capture it. One step (at 384 tokens, and at 16: the few-token path): forward and backward of two
adapted linears, then the clipped AdamW update of their adapters through a plan, whose bf16 copies
are the A and B the next forward reads. The graph is replayed three times, with eager work and a synchronisation between replays, and every replay
must equal the same step run eagerly, bit for bit (all kernels are deterministic).
"""
import numpy as np
import pytest

import workloads as wl
from gpu_helpers import dev, log

pytestmark = pytest.mark.gpu


def _setup(M):
    import torch
    import bit_nf4_quantised_amd as q
    r, s = 16, 2.0
    shapes = [(1024, 512), (768, 1024)]
    lins = []
    for i, (N, K) in enumerate(shapes):
        w = torch.from_numpy(wl.weight("single", 400 + i, N, K)).to(dev())
        g = wl.rng_for("single", 400 + i, "x")
        bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(dev()).to(torch.bfloat16)  # noqa: E731
        lin = dict(qw=q.quantize_weight(w),
                   x=bf(g.standard_normal((M, K))), dy=bf(g.standard_normal((M, N))),
                   pa=torch.from_numpy((g.standard_normal((r, K)) * 0.01).astype(np.float32)).to(dev()),
                   pb=torch.from_numpy((g.standard_normal((N, r)) * 0.01).astype(np.float32)).to(dev()),
                   y=torch.empty(M, N, dtype=torch.bfloat16, device=dev()),
                   u=torch.empty(M, r, dtype=torch.float32, device=dev()),
                   dx=torch.empty(M, K, dtype=torch.bfloat16, device=dev()),
                   dA=torch.empty(r, K, dtype=torch.float32, device=dev()),
                   dB=torch.empty(N, r, dtype=torch.float32, device=dev()),
                   ws=q.workspace(M, N, K, r))
        lin["A"] = lin["pa"].to(torch.bfloat16)
        lin["B"] = lin["pb"].to(torch.bfloat16)
        lins.append(lin)
    params = [t for l in lins for t in (l["pa"], l["pb"])]
    grads = [t for l in lins for t in (l["dA"], l["dB"])]
    copies = [t for l in lins for t in (l["A"], l["B"])]
    m = [torch.zeros_like(p) for p in params]
    v = [torch.zeros_like(p) for p in params]
    norm = torch.zeros(1, dtype=torch.float64, device=dev())
    plan = q.AdamWPlan(params, grads, m, v, copies, q.AdamWConfig(lr=1e-3))
    state = params + m + v + copies + [norm] + [l[k] for l in lins for k in ("y", "dx")]

    def step():
        for l in lins:
            q.qlora_linear_fwd(l["qw"], l["x"], l["A"], l["B"], s, l["y"], l["u"], ws=l["ws"])
            q.qlora_linear_bwd(l["qw"], l["x"], l["dy"], l["A"], l["B"], s, l["u"], l["dx"], l["dA"],
                               l["dB"], ws=l["ws"])
        plan.step(5, norm)

    return step, state


@pytest.mark.parametrize("M", [384, 16])
def test_training_step_replays_from_a_graph(M):
    # 384 tokens: the fused GEMMs; 16 tokens: the few-token forward and its epilogue, and the dX
    # GEMM with its contraction split into ranges and their ordered sum
    import torch
    log(f"[graph] M={M}")
    step, state = _setup(M)
    torch.cuda.synchronize()
    start = [t.clone() for t in state]
    eager = []
    for _ in range(3):
        step()
        torch.cuda.synchronize()
        eager.append([t.clone() for t in state])
    for t, t0 in zip(state, start):
        t.copy_(t0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(state, eager[rep])):
            assert torch.equal(got, want), f"replay {rep}: state tensor {i} differs from the eager step"
        junk = torch.randn(1 << 20, device=dev()).sum()   # eager work between replays
        float(junk)
        log(f"[graph] replay {rep} equals the eager step")
