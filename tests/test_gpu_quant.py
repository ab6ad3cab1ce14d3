"""GPU parity of quantise, double quantise and dequantise against the oracle: bit-exact.

Packed indices, first-level scales, E4M3 codes, second-level constants and dequantised bf16 values
must equal the oracle's byte for byte, on seeded synthetic weights of the workloads' shapes and
distributions and on adversarial blocks (zeros, signed zeros, subnormal scales, exact midpoint ties,
partial double-quantisation groups).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import dev, gpu_dequant, gpu_quantize, log, to_dev

pytestmark = pytest.mark.gpu


def check_weight_exact(w: np.ndarray, name: str):
    log(f"[quant] {name} shape={w.shape}")
    qw, packed, absmax, codes, c2 = gpu_quantize(w)
    p_ref, c1_ref = oracle.quantize(w)
    assert np.array_equal(absmax.view(np.uint32), c1_ref.view(np.uint32)), "absmax"
    bad = np.flatnonzero(packed != p_ref)
    assert bad.size == 0, f"packed differs at {bad.size} bytes, first {bad[:8]}"
    codes_ref, c2_ref = oracle.double_quant(c1_ref)
    assert np.array_equal(c2.view(np.uint32), c2_ref.view(np.uint32)), "c2"
    assert np.array_equal(codes, codes_ref), "scale codes"
    deq = gpu_dequant(qw)
    ref = oracle.dequant(p_ref, codes_ref, c2_ref, w.size)
    bad = np.flatnonzero(deq != ref)
    assert bad.size == 0, f"dequant differs at {bad.size} values, first {bad[:8]}"
    return qw


def test_single_linear_weight():
    w = wl.weight("single", 0, 4096, 4096, "gauss", 0.02)
    check_weight_exact(w, "single 4096x4096")


def _adversarial_weight():
    q = oracle.codebook().astype(np.float64)
    mids = (q[:-1] + q[1:]) / 2
    rng = np.random.default_rng(11)
    blocks = []
    for m in mids:                                  # exact midpoint ties where representable
        if np.float32(m) == m:
            b = np.clip(rng.normal(0, 0.1, 64), -0.49, 0.49).astype(np.float32)
            b[0] = 0.5
            b[1] = np.float32(0.5 * m)
            b[2] = np.nextafter(np.float32(0.5 * m), np.float32(1))
            b[3] = np.nextafter(np.float32(0.5 * m), np.float32(-1))
            blocks.append(b)
    # ties at every midpoint for scale c = 2^-3: c * m_i rounded down / up around the exact product
    for m in mids:
        b = np.zeros(64, np.float32)
        b[63] = np.float32(-0.125)
        t = 0.125 * m
        lo = np.float32(t)
        b[0:4] = [lo, np.nextafter(lo, np.float32(1)), np.nextafter(lo, np.float32(-1)), np.float32(-t)]
        blocks.append(b)
    blocks.append(np.zeros(64, np.float32))
    z = np.full(64, np.float32(-0.0)); z[7] = np.float32(3e-3); blocks.append(z)
    s = np.zeros(64, np.float32); s[17] = np.float32(1e-30); blocks.append(s)
    e = np.full(64, np.float32(0.01)); e[::2] = np.float32(-0.01); blocks.append(e)
    blocks.append((rng.standard_normal(64) * 1e-40).astype(np.float32))      # subnormal scale
    blocks.append((rng.standard_normal(64) * 1e-38).astype(np.float32))      # near the normal limit
    blocks.append((rng.standard_normal(64) * 1e30).astype(np.float32))
    blocks.append((rng.standard_normal(64) * 2.0 ** -100).astype(np.float32))
    big = rng.standard_t(2, 64).astype(np.float32); blocks.append(big)
    while len(blocks) % 16:
        blocks.append((rng.standard_normal(64) * 0.02).astype(np.float32))
    rows = len(blocks) // 16
    # 16 rows; each row holds `rows` blocks
    return np.stack(blocks).reshape(16, rows * 64)


def test_adversarial_blocks():
    check_weight_exact(_adversarial_weight(), "adversarial")


@pytest.mark.parametrize("kind,sigma", [("gauss_outlier", 0.015), ("student_t4", 0.015)])
def test_heavy_tailed_distributions(kind, sigma):
    w = wl.weight("llama65b" if kind == "gauss_outlier" else "llama70b", 50, 1024, 8192, kind, sigma)
    check_weight_exact(w, kind)


def test_stream_matrix():
    check_weight_exact(wl.stream_weight(0), "stream 4096x14336")


def test_ragged_flat_input_and_partial_group():
    import bit_nf4_quantised_amd as q
    numel = 64 * 1001                        # 1001 blocks: 3 full groups of 256 and one of 233
    w = (np.random.default_rng(12).standard_normal(numel) * 0.02).astype(np.float32)
    w[64 * 300:64 * 301] = 0.0
    log("[quant] ragged flat 64*1001")
    wd = to_dev(w)
    packed = torch.empty(numel // 2, dtype=torch.uint8, device=dev())
    absmax = torch.empty(numel // 64, dtype=torch.float32, device=dev())
    q.nf4_quantize(wd, packed, absmax)
    codes = torch.empty(numel // 64, dtype=torch.uint8, device=dev())
    c2 = torch.empty(4, dtype=torch.float32, device=dev())
    q.nf4_double_quant(absmax, codes, c2)
    torch.cuda.synchronize()
    p_ref, c1_ref = oracle.quantize(w)
    codes_ref, c2_ref = oracle.double_quant(c1_ref)
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    assert np.array_equal(absmax.cpu().numpy().view(np.uint32), c1_ref.view(np.uint32))
    assert np.array_equal(codes.cpu().numpy(), codes_ref)
    assert np.array_equal(c2.cpu().numpy().view(np.uint32), c2_ref.view(np.uint32))


@pytest.mark.parametrize("nblocks", [1, 255, 256, 257, 4097])
def test_double_quant_ties_and_sizes(nblocks):
    import bit_nf4_quantised_amd as q
    unit = oracle.e4m3_unit_values()
    mids = ((unit[:-1] + unit[1:]) / 2).astype(np.float32)
    rng = np.random.default_rng(nblocks)
    c1 = rng.uniform(0, 1, nblocks).astype(np.float32)
    c1[: min(nblocks, 56)] = mids[: min(nblocks, 56)]      # exact midpoints (group max 1.0 below)
    c1[::256] = 1.0
    if nblocks > 300:
        c1[256:512] = 0.0                                   # an all-zero group
    log(f"[dq] nblocks={nblocks}")
    cd = to_dev(c1)
    codes = torch.empty(nblocks, dtype=torch.uint8, device=dev())
    c2 = torch.empty((nblocks + 255) // 256, dtype=torch.float32, device=dev())
    q.nf4_double_quant(cd, codes, c2)
    torch.cuda.synchronize()
    codes_ref, c2_ref = oracle.double_quant(c1)
    assert np.array_equal(c2.cpu().numpy().view(np.uint32), c2_ref.view(np.uint32))
    assert np.array_equal(codes.cpu().numpy(), codes_ref)


def _e4m3_boundary_scales(c2: float, width: int = 8) -> np.ndarray:
    """Scales of groups whose maximum is c2: the float32 values within `width` ulps of c2 times every
    E4M3 value in [0, 1] and of c2 times every midpoint between neighbouring values, capped at c2;
    each group of 256 starts with c2 itself."""
    unit = oracle.e4m3_unit_values()
    pts = np.concatenate([unit, (unit[:-1] + unit[1:]) / 2])
    base = (pts * c2).astype(np.float32).view(np.uint32).astype(np.int64)
    cand = (base[:, None] + np.arange(-width, width + 1)[None, :]).reshape(-1)
    cand = cand[(cand >= 0) & (cand < 0x7F800000)].astype(np.uint32).view(np.float32)
    cand = np.unique(cand[cand <= np.float32(c2)])
    per = 255
    groups = -(-cand.size // per)
    out = np.zeros(groups * 256, np.float32)
    for g in range(groups):
        chunk = cand[g * per:(g + 1) * per]
        out[g * 256] = np.float32(c2)
        out[g * 256 + 1:g * 256 + 1 + chunk.size] = chunk
    return out


@pytest.mark.parametrize("c2", [1.0, 0.0213, 3.7e-5, 117.3, 2.0 ** -59, 1e-20])
def test_double_quant_at_every_code_boundary(c2):
    # scales within a few ulps of c2 times every E4M3 value and every midpoint between neighbours:
    # where the truncation to E4M3 and the one-fma midpoint decision are closest to going wrong
    # (c2 = 1e-20 takes the exact path for group maxima below 2^-60)
    import bit_nf4_quantised_amd as q
    c1 = _e4m3_boundary_scales(c2)
    log(f"[dq] boundary sweep c2={c2} scales={c1.size}")
    codes = torch.empty(c1.size, dtype=torch.uint8, device=dev())
    c2d = torch.empty(c1.size // 256, dtype=torch.float32, device=dev())
    q.nf4_double_quant(to_dev(c1), codes, c2d)
    torch.cuda.synchronize()
    codes_ref, c2_ref = oracle.double_quant(c1)
    assert np.array_equal(c2d.cpu().numpy().view(np.uint32), c2_ref.view(np.uint32))
    assert np.array_equal(codes.cpu().numpy(), codes_ref)
    # the batched kernel on the same scales, cut into three weights (the middle one ragged)
    cuts = [0, 768, 768 + 700, c1.size]
    parts = [to_dev(c1[a:b]) for a, b in zip(cuts, cuts[1:])]
    mcodes = [torch.empty(p.numel(), dtype=torch.uint8, device=dev()) for p in parts]
    mc2 = [torch.empty((p.numel() + 255) // 256, dtype=torch.float32, device=dev()) for p in parts]
    q.nf4_double_quant_many(parts, mcodes, mc2)
    torch.cuda.synchronize()
    for (a, b), mc, m2 in zip(zip(cuts, cuts[1:]), mcodes, mc2):
        cr, c2r = oracle.double_quant(c1[a:b])
        assert np.array_equal(mc.cpu().numpy(), cr)
        assert np.array_equal(m2.cpu().numpy().view(np.uint32), c2r.view(np.uint32))


def test_empty_input_is_a_noop():
    import bit_nf4_quantised_amd as q
    e = torch.empty(0, dtype=torch.float32, device=dev())
    q.nf4_quantize(e, torch.empty(0, dtype=torch.uint8, device=dev()), e)
    q.nf4_double_quant(e, torch.empty(0, dtype=torch.uint8, device=dev()),
                       torch.empty(0, dtype=torch.float32, device=dev()))
    torch.cuda.synchronize()


def test_quantise_is_deterministic():
    w = wl.weight("single", 3, 1024, 2048, "gauss", 0.02)
    a = gpu_quantize(w)
    b = gpu_quantize(w)
    for x, y in zip(a[1:], b[1:]):
        assert np.array_equal(x, y)
    assert np.array_equal(gpu_dequant(a[0]), gpu_dequant(b[0]))
