"""GPU parity of the adapter merge ("QLoRA, explained", Quality loss at merge time):
out = bf16(W~ + s B A) against the oracle's single rounding of the float64 sum.

Bar (the pages fix no precision for the merge; this one follows from the arithmetic): the GPU forms
B A in fp32 from exact bf16 products and adds it to W~ in fp32, so before the final bf16 rounding
its value is within about (r + 2) * 2^-24 (relative) of the exact sum, while a bf16 unit is 2^-8.
The two roundings can differ only for sums within that distance of a rounding tie: every element
must be within one bf16 unit of the oracle and at most 0.1 % may differ at all. A zero adapter must
give the dequantised weight bit for bit, and one-hot factors must touch exactly one element.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import bf16_to_dev, bits_from_dev, dev, gpu_dequant, gpu_quantize, log

pytestmark = pytest.mark.gpu


def _merge_gpu(qw, a_bits, b_bits, scale):
    import torch
    import bit_nf4_quantised_amd as q
    out = torch.empty(qw.N * qw.K, dtype=torch.int16, device=dev())
    q.qlora_merge(qw, bf16_to_dev(a_bits), bf16_to_dev(b_bits), scale, out)
    torch.cuda.synchronize()
    return bits_from_dev(out).reshape(qw.N, qw.K)


def _check(got, ref, name):
    g = got.astype(np.int32)
    r = ref.astype(np.int32)
    same_sign = (g & 0x8000) == (r & 0x8000)
    diff = np.abs(g - r)
    assert np.all(same_sign | (diff == 0)), f"{name}: sign differs"
    assert diff.max() <= 1, f"{name}: {int((diff > 1).sum())} values more than one bf16 unit off"
    frac = float((diff != 0).mean())
    log(f"[merge] {name}: {frac:.2e} of values one unit off")
    assert frac <= 1e-3, f"{name}: {frac:.2e} of values differ"


def _inputs(seed, n, k, r):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    a = wl.to_bf16_bits((rng.standard_normal((r, k)) * 0.01).astype(np.float32))
    b = wl.to_bf16_bits((rng.standard_normal((n, r)) * 0.01).astype(np.float32))
    return w, a, b


@pytest.mark.parametrize("n,k,r,s", [(400, 960, 16, 2.0), (256, 1024, 64, 0.25), (48, 64, 128, 0.5),
                                     (4096, 4096, 16, 2.0), (400, 960, 48, 1.0), (256, 1024, 80, 0.5),
                                     (208, 960, 96, 0.5), (400, 1088, 112, 0.25)])
def test_merge_matches_oracle(n, k, r, s):
    log(f"[merge] N={n} K={k} r={r} s={s}")
    w, a, b = _inputs(n + k + r, n, k, r)
    qw = gpu_quantize(w)[0]
    packed, c1 = oracle.quantize(w)
    codes, c2 = oracle.double_quant(c1)
    wt = oracle.dequant(packed, codes, c2, w.size).reshape(n, k)
    _check(_merge_gpu(qw, a, b, s), oracle.merge(wt, a, b, s), f"{n}x{k} r{r}")


def test_zero_adapter_gives_the_dequantised_weight():
    n, k, r = 272, 1088, 32
    w, a, _ = _inputs(3, n, k, r)
    b = np.zeros((n, r), dtype=np.uint16)
    qw = gpu_quantize(w)[0]
    assert np.array_equal(_merge_gpu(qw, a, b, 2.0), gpu_dequant(qw).reshape(n, k))


def test_one_hot_factors_touch_one_element():
    n, k, r = 64, 256, 16
    w = np.zeros((n, k), dtype=np.float32)
    a = np.zeros((r, k), dtype=np.uint16)
    b = np.zeros((n, r), dtype=np.uint16)
    a[9, 131] = wl.to_bf16_bits(np.float32([0.5]))[0]
    b[37, 9] = wl.to_bf16_bits(np.float32([0.25]))[0]
    qw = gpu_quantize(w)[0]
    got = _merge_gpu(qw, a, b, 4.0)
    want = np.zeros((n, k), dtype=np.uint16)
    want[37, 131] = wl.to_bf16_bits(np.float32([0.5]))[0]
    assert np.array_equal(got, want)


def test_merge_full_size_sampled_rows():
    """The 8192 x 28672 weight of the few-token forward, rank 16; the oracle checks 24 rows."""
    wk = wl.SKINNY
    lin = wk.linears[0]
    w, _, a, b, _ = wl.linear_inputs(wk, 0, lin, m=1)
    log(f"[merge] full size N={lin.n} K={lin.k} r={wk.r}")
    qw = gpu_quantize(w)[0]
    got = _merge_gpu(qw, a, b, wk.scale)
    packed, c1 = oracle.quantize(w)
    codes, c2 = oracle.double_quant(c1)
    rows = np.sort(np.random.default_rng(11).choice(lin.n, 24, replace=False))
    wt = oracle.dequant(packed, codes, c2, w.size).reshape(lin.n, lin.k)
    ref = oracle.merge(wt[rows], a, b[rows], wk.scale)
    _check(got[rows], ref, "full size rows")
