"""GPU parity of the adapter merge ("QLoRA, explained", Quality loss at merge time):
out = bf16(W~ + s B A), the exact value rounded once, against the oracle's single rounding of the
float64 sum. Bar: bit for bit. The kernel's fp32 sum goes through a rigorous near-tie test and the
values it cannot decide are recomputed exactly, so every case, including one built so that almost
every value sits near a rounding tie, must match exactly. A zero adapter must give the dequantised
weight bit for bit, and one-hot factors must touch exactly one element. The merged weight quantised
again from bf16 (nf4_quantize_bf16, then nf4_double_quant) must equal the oracle's quantisation of
the oracle's merge, bit for bit.
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
    diff = got != ref
    log(f"[merge] {name}: {int(diff.sum())} of {diff.size} values differ")
    assert not diff.any(), f"{name}: {int(diff.sum())} values differ from the exact rounding"


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


def test_merge_near_ties_everywhere():
    """Dequantised weight zero everywhere, B rows (c, -c, c, -c, ...) and, in every even column,
    A values equal in pairs (j = 2i, 2i + 1): the products cancel exactly there, the fp32 sum is 0
    and sits on the near-tie test's floor, so more than half of all values go through the exact
    recomputation (more than a wave's list holds at once for one tile)."""
    n, k, r, s = 256, 1024, 16, 2.0
    log(f"[merge] near ties N={n} K={k} r={r}")
    rng = np.random.default_rng(5)
    w = np.zeros((n, k), dtype=np.float32)
    af = (rng.standard_normal((r, k)) * 0.01).astype(np.float32)
    af[1::2, 0::2] = af[0::2, 0::2]
    a = wl.to_bf16_bits(af)
    sign = np.where(np.arange(r) % 2 == 1, -1.0, 1.0)
    mag = (0.01 * (1.0 + rng.random(n))).astype(np.float32)
    b = wl.to_bf16_bits((sign[None, :] * mag[:, None]).astype(np.float32))
    qw = gpu_quantize(w)[0]
    wt = np.zeros((n, k), dtype=np.uint16)
    _check(_merge_gpu(qw, a, b, s), oracle.merge(wt, a, b, s), "near ties")


@pytest.mark.parametrize("n,k,r,s", [(400, 960, 16, 2.0), (256, 1088, 64, 0.25)])
def test_merged_weight_requantised_from_bf16(n, k, r, s):
    import torch
    import bit_nf4_quantised_amd as q
    log(f"[merge] re-quantise N={n} K={k} r={r}")
    w, a, b = _inputs(7 * n + k, n, k, r)
    qw = gpu_quantize(w)[0]
    merged = torch.empty(n * k, dtype=torch.int16, device=dev())
    q.qlora_merge(qw, bf16_to_dev(a), bf16_to_dev(b), s, merged)
    packed = torch.empty(n * k // 2, dtype=torch.uint8, device=dev())
    absmax = torch.empty(n * k // 64, dtype=torch.float32, device=dev())
    q.nf4_quantize_bf16(merged, packed, absmax)
    nb = n * k // 64
    codes = torch.empty(nb, dtype=torch.uint8, device=dev())
    c2 = torch.empty((nb + 255) // 256, dtype=torch.float32, device=dev())
    q.nf4_double_quant(absmax, codes, c2)
    torch.cuda.synchronize()
    p0, c10 = oracle.quantize(w)
    k0, c20 = oracle.double_quant(c10)
    wt = oracle.dequant(p0, k0, c20, w.size).reshape(n, k)
    merged_ref = oracle.merge(wt, a, b, s)
    w2 = oracle.f32_from_bf16_bits(merged_ref.reshape(-1)).reshape(n, k)
    p_ref, c1_ref = oracle.quantize(w2)
    k_ref, c2_ref = oracle.double_quant(c1_ref)
    assert np.array_equal(bits_from_dev(merged).reshape(n, k), merged_ref)
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    assert np.array_equal(absmax.cpu().numpy().view(np.uint32), np.asarray(c1_ref, np.float32).view(np.uint32))
    assert np.array_equal(codes.cpu().numpy(), k_ref)
    assert np.array_equal(c2.cpu().numpy().view(np.uint32), np.asarray(c2_ref, np.float32).view(np.uint32))
