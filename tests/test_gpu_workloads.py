"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

Every linear of the layer sets is quantised on the GPU and compared bit-exactly with the oracle
(packed indices, scales, codes, constants, dequantised bf16), then run forward and backward at the
full token count; the oracle computes a sample of outputs one by one: rows of y and dX, columns of
dA, rows of dB. The skinny forward is checked in full at 1, 4 and 16 tokens.
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


@pytest.mark.parametrize("name,li", CASES)
def test_layer_linear(name, li):
    wk = wl.WORKLOADS[name]
    lin = wk.linears[li]
    log(f"[workload] {name}.{lin.name} N={lin.n} K={lin.k} M={wk.m} r={wk.r}")
    w, x, a, b, dy = wl.linear_inputs(wk, li, lin)
    qw, packed, absmax, codes, c2 = gpu_quantize(w)
    p_ref, c1_ref, codes_ref, c2_ref = _oracle_quant(w)
    assert np.array_equal(absmax.view(np.uint32), c1_ref.view(np.uint32))
    assert np.array_equal(packed, p_ref)
    assert np.array_equal(codes, codes_ref)
    assert np.array_equal(c2.view(np.uint32), c2_ref.view(np.uint32))
    wt = oracle.dequant(p_ref, codes_ref, c2_ref, w.size).reshape(lin.n, lin.k)
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
