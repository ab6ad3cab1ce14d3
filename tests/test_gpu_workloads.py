"""GPU parity at the workloads' full sizes, in the launch configurations the benchmark times.

Every linear of the layer sets is quantised on the GPU and compared bit-exactly with the oracle
(packed indices, scales, codes, constants, dequantised bf16), then run forward and backward at the
full token count; the oracle computes a sample of outputs one by one: rows of y and dX, columns of
dA, rows of dB. The linears that share their input (q, k, v and gate, up) also run as the benchmark
runs them, as one grouped forward and one grouped backward on the first member's x, each output
sampled against the oracle's linear on that linear's own weight. The skinny forward is checked in
full at 1, 4 and 16 tokens.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import assert_close, f64_from_bits, gpu_dequant, gpu_fwd_bwd, gpu_quantize, log

pytestmark = pytest.mark.gpu

# every linear of the 8B set; the distinct shapes (q, k, gate, down) of the 65B and 70B sets
CASES = ([("llama8b", i) for i in range(7)] + [("llama65b", i) for i in (0, 1, 4, 6)]
         + [("llama70b", i) for i in (0, 1, 4, 6)])


def _oracle_quant(w):
    packed, c1 = oracle.quantize(w)
    codes, c2 = oracle.double_quant(c1)
    return packed, c1, codes, c2


# members of the groups the benchmark launches as one: their inputs and the oracle's dequantised
# weight, kept for the grouped cases below (the single-linear cases compute them first)
GROUPS = (("q", "k", "v"), ("gate", "up"))
_MEMBERS = {n for g in GROUPS for n in g}
_CACHE = {}


def _linear_data(name, li):
    key = (name, li)
    if key in _CACHE:
        return _CACHE[key]
    wk = wl.WORKLOADS[name]
    lin = wk.linears[li]
    w, x, a, b, dy = wl.linear_inputs(wk, li, lin)
    packed, c1, codes, c2 = _oracle_quant(w)
    wt = oracle.dequant(packed, codes, c2, w.size).reshape(lin.n, lin.k)
    out = (w, x, a, b, dy, packed, c1, codes, c2, wt)
    if lin.name in _MEMBERS:
        _CACHE[key] = out
    return out


@pytest.mark.parametrize("name,li", CASES)
def test_layer_linear(name, li):
    wk = wl.WORKLOADS[name]
    lin = wk.linears[li]
    log(f"[workload] {name}.{lin.name} N={lin.n} K={lin.k} M={wk.m} r={wk.r}")
    w, x, a, b, dy, p_ref, c1_ref, codes_ref, c2_ref, wt = _linear_data(name, li)
    qw, packed, absmax, codes, c2 = gpu_quantize(w)
    assert np.array_equal(absmax.view(np.uint32), c1_ref.view(np.uint32))
    assert np.array_equal(packed, p_ref)
    assert np.array_equal(codes, codes_ref)
    assert np.array_equal(c2.view(np.uint32), c2_ref.view(np.uint32))
    del p_ref, c1_ref
    assert np.array_equal(gpu_dequant(qw).reshape(lin.n, lin.k), wt)

    y, u, dx, dA, dB = gpu_fwd_bwd(qw, x, a, b, dy, wk.scale)
    rng = np.random.default_rng(li)
    rows = np.sort(rng.choice(wk.m, 12, replace=False))
    acols = np.sort(rng.choice(lin.k, 64, replace=False))
    brows = np.sort(rng.choice(lin.n, 64, replace=False))
    yr, ur = oracle.linear_fwd(x[rows], wt, a, b, wk.scale)
    assert_close("y rows", f64_from_bits(y[rows]), yr)
    assert_close("u rows", u[rows], ur)
    dxr, dar, dbr = oracle.linear_bwd_sampled(x, dy, wt, a, b, wk.scale, rows, acols, brows)
    assert_close("dX rows", f64_from_bits(dx[rows]), dxr)
    assert_close("dA cols", dA[:, acols], dar)
    assert_close("dB rows", dB[brows], dbr)


@pytest.mark.parametrize("name,grp", [(n, g) for n in ("llama8b", "llama65b", "llama70b") for g in GROUPS])
def test_layer_group(name, grp):
    import torch
    import bit_nf4_quantised_amd as q
    from gpu_helpers import bf16_to_dev, bits_from_dev, dev
    wk = wl.WORKLOADS[name]
    idx = [next(i for i, lin in enumerate(wk.linears) if lin.name == n) for n in grp]
    lins = [wk.linears[i] for i in idx]
    log(f"[workload] {name} group {'+'.join(grp)} N={[lin.n for lin in lins]} K={lins[0].k} M={wk.m} r={wk.r}")
    data = [_linear_data(name, i) for i in idx]
    x = data[0][1]   # the members share the first member's x
    qws = [gpu_quantize(d[0])[0] for d in data]
    M, K, r, s = wk.m, lins[0].k, wk.r, wk.scale
    X = bf16_to_dev(x)
    As = [bf16_to_dev(d[2]) for d in data]
    Bs = [bf16_to_dev(d[3]) for d in data]
    ys = [torch.empty(M, lin.n, dtype=torch.int16, device=dev()) for lin in lins]
    us = [torch.empty(M, r, dtype=torch.float32, device=dev()) for _ in lins]
    dxs = [torch.empty(M, K, dtype=torch.int16, device=dev()) for _ in lins]
    dAs = [torch.empty(r, K, dtype=torch.float32, device=dev()) for _ in lins]
    dBs = [torch.empty(lin.n, r, dtype=torch.float32, device=dev()) for lin in lins]
    q.qlora_linear_fwd_group(qws, X, As, Bs, s, ys, us)
    q.qlora_linear_bwd_group(qws, X, [bf16_to_dev(d[4]) for d in data], As, Bs, s, us, dxs, dAs, dBs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(idx[0] + 100)
    rows = np.sort(rng.choice(M, 12, replace=False))
    acols = np.sort(rng.choice(K, 64, replace=False))
    for j, (lin, d) in enumerate(zip(lins, data)):
        _, _, a, b, dy, _, _, _, _, wt = d
        brows = np.sort(rng.choice(lin.n, 64, replace=False))
        yr, ur = oracle.linear_fwd(x[rows], wt, a, b, s)
        assert_close(f"{lin.name} y rows", f64_from_bits(bits_from_dev(ys[j])[rows]), yr)
        assert_close(f"{lin.name} u rows", us[j].cpu().numpy()[rows], ur)
        dxr, dar, dbr = oracle.linear_bwd_sampled(x, dy, wt, a, b, s, rows, acols, brows)
        assert_close(f"{lin.name} dX rows", f64_from_bits(bits_from_dev(dxs[j])[rows]), dxr)
        assert_close(f"{lin.name} dA cols", dAs[j].cpu().numpy()[:, acols], dar)
        assert_close(f"{lin.name} dB rows", dBs[j].cpu().numpy()[brows], dbr)
    del qws, ys, us, dxs, dAs, dBs
    torch.cuda.empty_cache()
    for i in idx:
        _CACHE.pop((name, i), None)


@pytest.mark.parametrize("M", wl.SKINNY_MS)
def test_skinny_forward(M):
    wk = wl.SKINNY
    lin = wk.linears[0]
    log(f"[workload] skinny M={M} N={lin.n} K={lin.k}")
    w, x, a, b, dy = wl.linear_inputs(wk, 0, lin, m=M)
    import torch
    import bit_nf4_quantised_amd as q
    from gpu_helpers import bf16_to_dev, bits_from_dev, dev
    qw = gpu_quantize(w)[0]
    y = torch.empty(M, lin.n, dtype=torch.int16, device=dev())
    u = torch.empty(M, wk.r, dtype=torch.float32, device=dev())
    q.qlora_linear_fwd(qw, bf16_to_dev(x), bf16_to_dev(a), bf16_to_dev(b), wk.scale, y, u)
    torch.cuda.synchronize()
    p_ref, c1_ref, codes_ref, c2_ref = _oracle_quant(w)
    assert np.array_equal(qw.packed.cpu().numpy(), p_ref)
    wt = oracle.dequant(p_ref, codes_ref, c2_ref, w.size).reshape(lin.n, lin.k)
    yr, ur = oracle.linear_fwd(x, wt, a, b, wk.scale)
    assert_close("y", f64_from_bits(bits_from_dev(y)), yr)
    assert_close("u", u.cpu().numpy(), ur)


@pytest.mark.parametrize("M", [1, 16])
def test_skinny_forward_fp32_scales(M):
    # the few-token forward on the same full-size weight keeping its fp32 absmax (no double
    # quantisation): the four-row kernel at M = 1, the 16-row kernel at M = 16
    wk = wl.SKINNY
    lin = wk.linears[0]
    log(f"[workload] skinny fp32 scales M={M} N={lin.n} K={lin.k}")
    w, x, a, b, dy = wl.linear_inputs(wk, 0, lin, m=M)
    import torch
    import bit_nf4_quantised_amd as q
    from gpu_helpers import bf16_to_dev, bits_from_dev, dev, to_dev
    qw = q.quantize_weight(to_dev(w.astype(np.float32)), double_quant=False)
    y = torch.empty(M, lin.n, dtype=torch.int16, device=dev())
    u = torch.empty(M, wk.r, dtype=torch.float32, device=dev())
    q.qlora_linear_fwd(qw, bf16_to_dev(x), bf16_to_dev(a), bf16_to_dev(b), wk.scale, y, u)
    torch.cuda.synchronize()
    p_ref, c1_ref = oracle.quantize(w)
    assert np.array_equal(qw.packed.cpu().numpy(), p_ref)
    assert np.array_equal(qw.absmax.cpu().numpy(), c1_ref.astype(np.float32))
    wt = oracle.dequant_blocks(p_ref, c1_ref, oracle.codebook(), 64, w.size).reshape(lin.n, lin.k)
    yr, ur = oracle.linear_fwd(x, wt, a, b, wk.scale)
    assert_close("y", f64_from_bits(bits_from_dev(y)), yr)
    assert_close("u", u.cpu().numpy(), ur)
