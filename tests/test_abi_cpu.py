"""Host-side checks of the C ABI: the library loads, exports every call the header declares, and
rejects bad arguments with the documented status before touching the GPU. No kernel runs here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
q = pytest.importorskip("bit_nf4_quantised_amd")
lib = q.lib

FAKE = 0x100000          # an aligned, never-dereferenced address
MISALIGNED = FAKE + 4


def declared_functions():
    src = open(os.path.join(ROOT, "include", "qlora_nf4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(q.EXPORTED), names
    for n in names:
        assert hasattr(lib, n)


def test_codebook_constants_equal_oracle():
    got = np.array(q.nf4_codebook(), dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), oracle.codebook().view(np.uint32))


def test_storage_bytes():
    for numel in (0, 64, 64 * 300, 4096 * 4096, 8192 * 28672):
        nb = numel // 64
        want = numel // 2 + nb + 4 * ((nb + 255) // 256)
        assert q.nf4_storage_bytes(numel) == want
    assert q.nf4_storage_bytes(65) == -1 and q.nf4_storage_bytes(-64) == -1
    # at scale, bits per parameter match the page's 4.127
    n = 8192 * 28672
    assert round(8 * q.nf4_storage_bytes(n) / n, 3) == round(oracle.storage_bits(64), 3)


def test_workspace_bytes():
    assert q.qlora_workspace_bytes(2048, 4096, 4096, 16) > 0
    assert q.qlora_workspace_bytes(1, 8192, 28672, 16) > 0
    assert q.qlora_workspace_bytes(16, 4096, 4096, 8) == 0          # bad rank
    assert q.qlora_workspace_bytes(16, 4095, 4096, 16) == 0         # N % 16
    assert q.qlora_workspace_bytes(16, 4096, 4000, 16) == 0         # K % 64


def test_status_strings():
    for s in range(7):
        assert lib.nf4_status_string(s)
    assert b"unknown" in lib.nf4_status_string(99)


def test_quantize_validation():
    assert lib.nf4_quantize(FAKE, 65, FAKE, FAKE, None) == q.NF4_ERR_SHAPE
    assert lib.nf4_quantize(FAKE, -64, FAKE, FAKE, None) == q.NF4_ERR_SHAPE
    assert lib.nf4_quantize(None, 64, FAKE, FAKE, None) == q.NF4_ERR_NULL
    assert lib.nf4_quantize(MISALIGNED, 64, FAKE, FAKE, None) == q.NF4_ERR_ALIGN
    assert lib.nf4_quantize(None, 0, None, None, None) == q.NF4_OK      # empty input: nothing to do


def test_quantize_bf16_validation():
    assert lib.nf4_quantize_bf16(FAKE, 65, FAKE, FAKE, None) == q.NF4_ERR_SHAPE
    assert lib.nf4_quantize_bf16(FAKE, -64, FAKE, FAKE, None) == q.NF4_ERR_SHAPE
    assert lib.nf4_quantize_bf16(None, 64, FAKE, FAKE, None) == q.NF4_ERR_NULL
    assert lib.nf4_quantize_bf16(FAKE, 64, FAKE, None, None) == q.NF4_ERR_NULL
    assert lib.nf4_quantize_bf16(MISALIGNED, 64, FAKE, FAKE, None) == q.NF4_ERR_ALIGN
    assert lib.nf4_quantize_bf16(None, 0, None, None, None) == q.NF4_OK   # empty input: nothing to do


def test_double_quant_validation():
    assert lib.nf4_double_quant(FAKE, -1, FAKE, FAKE, None) == q.NF4_ERR_SHAPE
    assert lib.nf4_double_quant(FAKE, 10, None, FAKE, None) == q.NF4_ERR_NULL
    assert lib.nf4_double_quant(FAKE, 10, FAKE, MISALIGNED, None) == q.NF4_ERR_ALIGN
    assert lib.nf4_double_quant(None, 0, None, None, None) == q.NF4_OK


def _w(N=4096, K=4096, packed=FAKE):
    return q.CNF4Weight(packed, FAKE, FAKE, N, K)


def test_dequant_validation():
    assert lib.nf4_dequant(None, FAKE, None) == q.NF4_ERR_NULL
    assert lib.nf4_dequant(ctypes.byref(_w(packed=None)), FAKE, None) == q.NF4_ERR_NULL
    assert lib.nf4_dequant(ctypes.byref(_w(N=4090)), FAKE, None) == q.NF4_ERR_SHAPE
    assert lib.nf4_dequant(ctypes.byref(_w(K=4000)), FAKE, None) == q.NF4_ERR_SHAPE
    assert lib.nf4_dequant(ctypes.byref(_w(N=0)), FAKE, None) == q.NF4_ERR_SHAPE
    assert lib.nf4_dequant(ctypes.byref(_w(packed=MISALIGNED)), FAKE, None) == q.NF4_ERR_ALIGN
    assert lib.nf4_dequant(ctypes.byref(_w()), None, None) == q.NF4_ERR_NULL


def test_weight_scale_kinds():
    # exactly one kind of scales: double quantised, or fp32 absmax
    both = q.CNF4Weight(FAKE, FAKE, FAKE, 4096, 4096, FAKE)
    assert lib.nf4_dequant(ctypes.byref(both), FAKE, None) == q.NF4_ERR_NULL
    half = q.CNF4Weight(FAKE, None, FAKE, 4096, 4096, None)
    assert lib.nf4_dequant(ctypes.byref(half), FAKE, None) == q.NF4_ERR_NULL
    mis = q.CNF4Weight(FAKE, None, None, 4096, 4096, MISALIGNED)
    assert lib.nf4_dequant(ctypes.byref(mis), FAKE, None) == q.NF4_ERR_ALIGN
    f32s = q.CNF4Weight(FAKE, None, None, 4096, 4096, FAKE)
    assert lib.qlora_merge(ctypes.byref(f32s), FAKE, FAKE, 16, 2.0, FAKE, None) == q.NF4_ERR_SHAPE


def test_weight_codebook_validation():
    # the codebook field of the weight: 0 NF4, 1 FP4, 2 INT4; anything else is a shape error in
    # every call that takes a weight, before any HIP call
    for bad in (-1, 3, 1 << 20):
        w = ctypes.byref(q.CNF4Weight(FAKE, FAKE, FAKE, 4096, 4096, None, bad))
        assert lib.nf4_dequant(w, FAKE, None) == q.NF4_ERR_SHAPE
        assert lib.qlora_merge(w, FAKE, FAKE, 16, 2.0, FAKE, None) == q.NF4_ERR_SHAPE
        assert lib.qlora_linear_fwd(w, FAKE, 64, FAKE, FAKE, 16, 2.0, FAKE, None, FAKE, 1 << 30,
                                    None) == q.NF4_ERR_SHAPE
        assert lib.qlora_linear_fwd_noalloc(w, FAKE, 64, FAKE, FAKE, 16, 2.0, FAKE, None,
                                            None) == q.NF4_ERR_SHAPE
        assert lib.qlora_linear_fwd_recompute(w, FAKE, 64, FAKE, FAKE, 16, 2.0, FAKE, FAKE, FAKE,
                                              1 << 30, None) == q.NF4_ERR_SHAPE
        assert lib.qlora_linear_bwd(w, FAKE, FAKE, 64, FAKE, FAKE, 16, 2.0, FAKE, FAKE, FAKE, FAKE,
                                    0, FAKE, 1 << 30, None) == q.NF4_ERR_SHAPE
    # the binding names the codebooks and passes the field through
    assert q.NF4Weight(None, None, None, 64, 64, codebook="fp4").c_struct().codebook == 1
    assert q.NF4Weight(None, None, None, 64, 64, codebook=2).c_struct().codebook == 2
    assert q.NF4Weight(None, None, None, 64, 64).c_struct().codebook == 0
    assert q.CNF4Weight(FAKE, FAKE, FAKE, 64, 64).codebook == 0


def test_merge_validation():
    w = ctypes.byref(_w())
    assert lib.qlora_merge(None, FAKE, FAKE, 16, 2.0, FAKE, None) == q.NF4_ERR_NULL
    assert lib.qlora_merge(ctypes.byref(_w(K=4000)), FAKE, FAKE, 16, 2.0, FAKE, None) == q.NF4_ERR_SHAPE
    assert lib.qlora_merge(w, FAKE, FAKE, 8, 2.0, FAKE, None) == q.NF4_ERR_RANK
    assert lib.qlora_merge(w, FAKE, FAKE, 144, 2.0, FAKE, None) == q.NF4_ERR_RANK
    assert lib.qlora_merge(w, None, FAKE, 16, 2.0, FAKE, None) == q.NF4_ERR_NULL
    assert lib.qlora_merge(w, FAKE, None, 16, 2.0, FAKE, None) == q.NF4_ERR_NULL
    assert lib.qlora_merge(w, FAKE, FAKE, 16, 2.0, None, None) == q.NF4_ERR_NULL
    assert lib.qlora_merge(w, MISALIGNED, FAKE, 16, 2.0, FAKE, None) == q.NF4_ERR_ALIGN
    assert lib.qlora_merge(w, FAKE, FAKE, 16, 2.0, MISALIGNED, None) == q.NF4_ERR_ALIGN


def test_fwd_validation():
    w = ctypes.byref(_w())
    ws = q.qlora_workspace_bytes(64, 4096, 4096, 16)
    f = lib.qlora_linear_fwd
    assert f(w, FAKE, 64, FAKE, FAKE, 8, 2.0, FAKE, None, FAKE, ws, None) == q.NF4_ERR_RANK
    assert f(w, FAKE, 64, FAKE, FAKE, 24, 2.0, FAKE, None, FAKE, ws, None) == q.NF4_ERR_RANK
    assert f(w, FAKE, 64, FAKE, FAKE, 256, 2.0, FAKE, None, FAKE, ws, None) == q.NF4_ERR_RANK
    assert f(w, FAKE, -1, FAKE, FAKE, 16, 2.0, FAKE, None, FAKE, ws, None) == q.NF4_ERR_SHAPE
    assert f(w, None, 64, FAKE, FAKE, 16, 2.0, FAKE, None, FAKE, ws, None) == q.NF4_ERR_NULL
    assert f(w, FAKE, 64, FAKE, FAKE, 16, 2.0, None, None, FAKE, ws, None) == q.NF4_ERR_NULL
    assert f(w, FAKE, 64, MISALIGNED, FAKE, 16, 2.0, FAKE, None, FAKE, ws, None) == q.NF4_ERR_ALIGN
    assert f(w, FAKE, 64, FAKE, FAKE, 16, 2.0, FAKE, None, None, ws, None) == q.NF4_ERR_WORKSPACE
    assert f(w, FAKE, 64, FAKE, FAKE, 16, 2.0, FAKE, None, FAKE, 16, None) == q.NF4_ERR_WORKSPACE
    assert f(w, FAKE, 0, FAKE, FAKE, 16, 2.0, FAKE, None, None, 0, None) == q.NF4_OK
    assert f(None, FAKE, 64, FAKE, FAKE, 16, 2.0, FAKE, None, FAKE, ws, None) == q.NF4_ERR_NULL


def _skinny_fwd_bytes(M, N, K, r):
    """Forward workspace of the few-token path, from its documented plan: M <= 4 takes 64-row
    blocks and 2048-column steps, larger M 256-row blocks and 512-column steps; the row blocks
    times the k splits (the items) fill 256 workgroups at most, every item leaves one partial sum
    of u, and u plus the partials come first."""
    rows, step = (64, 2048) if M <= 4 else (256, 512)
    nsteps = -(-K // step)
    blocks = -(-N // rows)
    want = min(max(256 // blocks, 1), nsteps)
    sub = -(-nsteps // want)
    splits = -(-nsteps // sub)
    part = ((splits * M * N + 3) // 4) * 4 + splits * blocks * M * r
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    return up(M * r * 4) + up(part * 4)


@pytest.mark.parametrize("M,N,K,r", [(1, 8192, 28672, 16), (4, 8192, 28672, 16), (5, 8192, 28672, 16),
                                     (16, 8192, 28672, 16), (3, 1040, 1088, 128), (4, 96, 4160, 32),
                                     (1, 16, 2048, 64), (2, 14336, 4096, 64)])
def test_skinny_workspace_follows_the_plan(M, N, K, r):
    need = _skinny_fwd_bytes(M, N, K, r)
    assert q.qlora_workspace_bytes(M, N, K, r) >= need
    # one byte less than the plan's partial sums is refused before any launch
    w = ctypes.byref(_w(N=N, K=K))
    assert lib.qlora_linear_fwd(w, FAKE, M, FAKE, FAKE, r, 2.0, FAKE, None, FAKE, need - 1, None) == \
        q.NF4_ERR_WORKSPACE


def _few_tile_ranges(tiles, steps, bm):
    """Contraction ranges of 128- and 64-row tiles: none below 8 steps; else as many as keep the
    workgroups within one round of 256 CUs, at most 4 (8 for 64-row tiles), and at most
    max(2, steps // 8)."""
    if steps < 8:
        return 1
    return max(1, min(8 if bm == 64 else 4, max(2, steps // 8), 256 // tiles))


def _gemm_fwd_bytes(M, N, K, r):
    """Forward workspace of the fused-GEMM path (M > 16), from its documented plan: 256-row tiles
    when there are at least 192 of them, with the tiles past the last whole round of 256 CUs cut
    into 2..4 contraction ranges (tile-major partial sums of 256 x 128 per piece); else, above 128
    tokens, 256-row tiles with ks = 2..4 contraction ranges of at least 8 steps when that makes at
    least 192 workgroups; else 128-row tiles (64 at most 64 tokens) with _few_tile_ranges ranges.
    A uniform split leaves ks x M x N fp32 partial sums; u comes first. (At rank 16 the adapter's u
    needs no partial sums of its own.)"""
    gx, steps = -(-N // 128), -(-K // 64)
    t256 = gx * -(-M // 256)
    ks, part = 1, 0
    if M > 128 and t256 >= 192:
        # the tail: the tiles past the last whole round of 256 CUs, cut into 2..4 ranges
        rem = t256 % 256
        s = min(4, 256 // rem, steps // 8) if rem else 0
        if t256 > 256 and rem and s >= 2 and (t256 - rem) % 8 == 0 and (rem * s) % 8 == 0:
            ks, part = s, s * rem * 256 * 128
    elif M > 128 and min(4, steps // 8, -(-256 // t256)) > 1 and t256 * min(4, steps // 8, -(-256 // t256)) >= 192:
        ks = min(4, steps // 8, -(-256 // t256))
        part = ks * M * N
    else:
        bm = 64 if M <= 64 else 128
        ks = _few_tile_ranges(gx * -(-M // bm), steps, bm)
        part = ks * M * N if ks > 1 else 0
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    return up(M * r * 4) + (up(part * 4) if part else 0), ks


@pytest.mark.parametrize("M,N,K,ks", [(2048, 1024, 4096, 4), (4096, 1024, 8192, 2), (1500, 1040, 2112, 4),
                                      (2048, 4096, 4096, 1), (300, 400, 960, 2), (1800, 128, 14336, 4),
                                      (2048, 14336, 4096, 2), (300, 16512, 2048, 4), (4096, 28672, 8192, 1),
                                      (40, 4096, 2048, 4), (64, 4096, 4096, 8), (100, 256, 1024, 2),
                                      (40, 256, 512, 2), (300, 19200, 960, 1)])
def test_gemm_workspace_follows_the_plan(M, N, K, ks):
    need, plan_ks = _gemm_fwd_bytes(M, N, K, 16)
    assert plan_ks == ks
    assert q.qlora_workspace_bytes(M, N, K, 16) >= need
    if ks > 1:   # one byte less than u plus the partial sums is refused before any launch
        w = ctypes.byref(_w(N=N, K=K))
        assert lib.qlora_linear_fwd(w, FAKE, M, FAKE, FAKE, 16, 2.0, FAKE, None, FAKE, need - 1, None) == \
            q.NF4_ERR_WORKSPACE


def _dx_plan_ks(M, N, K):
    """Contraction ranges of the dX GEMM, from its documented plan: 256-row tiles when there are at
    least 192 of them (their tail aside, never a uniform split); else 128-row tiles (64 at most 64
    tokens) with _few_tile_ranges ranges."""
    gx, steps = -(-K // 128), -(-N // 64)
    if M > 128 and gx * -(-M // 256) >= 192:
        return 1
    bm = 128 if M > 64 else 64
    return _few_tile_ranges(gx * -(-M // bm), steps, bm)


@pytest.mark.parametrize("M,N,K,ks", [(16, 4096, 28672, 1), (16, 4096, 4096, 8), (100, 2048, 1024, 4),
                                      (40, 1040, 2112, 2), (16, 416, 1024, 1), (2048, 4096, 4096, 1)])
def test_dx_workspace_follows_the_plan(M, N, K, ks):
    assert _dx_plan_ks(M, N, K) == ks
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    part = ks * M * K * 4 if ks > 1 else 0
    assert q.qlora_workspace_bytes(M, N, K, 16) >= up(M * 16 * 4) + (up(part) if part else 0)
    if (M, N, K) == (16, 4096, 4096):
        # the dX partial sums are the backward's largest partials here, so its workspace is v plus
        # them exactly: one byte less is refused before any launch
        need = up(M * 16 * 4) + up(part)
        w = ctypes.byref(_w(N=N, K=K))
        assert lib.qlora_linear_bwd(w, FAKE, FAKE, M, FAKE, FAKE, 16, 2.0, FAKE, FAKE, FAKE, FAKE, 0, FAKE,
                                    need - 1, None) == q.NF4_ERR_WORKSPACE


@pytest.mark.parametrize("M,N,K", [(1, 8192, 28672), (5, 4096, 512), (16, 4096, 512), (16, 8192, 28672)])
def test_fp32_scale_few_token_workspace_follows_the_plan(M, N, K):
    # a weight with fp32 scales takes the few-token path at 1..16 tokens like a double-quantised
    # one, with the same plan: one byte less than its partial sums is refused before any launch
    r = 16
    need = _skinny_fwd_bytes(M, N, K, r)
    assert q.qlora_workspace_bytes(M, N, K, r) >= need
    w = q.CNF4Weight(FAKE, None, None, N, K)
    w.absmax = FAKE
    assert lib.qlora_linear_fwd(ctypes.byref(w), FAKE, M, FAKE, FAKE, r, 2.0, FAKE, None, FAKE, need - 1, None) == \
        q.NF4_ERR_WORKSPACE


def test_group_validation():
    f = lib.qlora_linear_fwd_group
    P = ctypes.c_void_p
    a, b, c = q.CNF4Weight(FAKE, FAKE, FAKE, 4096, 4096), q.CNF4Weight(FAKE, FAKE, FAKE, 1024, 4096), \
        q.CNF4Weight(FAKE, FAKE, FAKE, 1024, 2048)
    ptrs = lambda *ws: (P * len(ws))(*[ctypes.addressof(w) for w in ws])  # noqa: E731
    fake = lambda n: (P * n)(*([FAKE] * n))  # noqa: E731
    n2 = (ctypes.c_int64 * 2)(4096, 1024)
    need = q.lib.qlora_workspace_bytes_group(2, n2, 2048, 4096, 16)
    assert need > 0
    # (no call with valid arguments: it would launch kernels on the fake pointers)
    assert f(0, ptrs(a, b), FAKE, 2048, fake(2), fake(2), 16, 2.0, fake(2), None, FAKE, need, None) == q.NF4_ERR_SHAPE
    assert f(5, ptrs(a, b, a, b, a), FAKE, 2048, fake(5), fake(5), 16, 2.0, fake(5), None, FAKE, need, None) == \
        q.NF4_ERR_SHAPE
    assert f(2, None, FAKE, 2048, fake(2), fake(2), 16, 2.0, fake(2), None, FAKE, need, None) == q.NF4_ERR_NULL
    assert f(2, ptrs(a, b), FAKE, 2048, None, fake(2), 16, 2.0, fake(2), None, FAKE, need, None) == q.NF4_ERR_NULL
    # weights that differ in K, or in the kind of scales
    assert f(2, ptrs(a, c), FAKE, 2048, fake(2), fake(2), 16, 2.0, fake(2), None, FAKE, need, None) == \
        q.NF4_ERR_SHAPE
    d = q.CNF4Weight(FAKE, None, None, 1024, 4096, FAKE)
    assert f(2, ptrs(a, d), FAKE, 2048, fake(2), fake(2), 16, 2.0, fake(2), None, FAKE, need, None) == \
        q.NF4_ERR_SHAPE
    e = q.CNF4Weight(FAKE, FAKE, FAKE, 1024, 4096, None, 1)
    assert f(2, ptrs(a, e), FAKE, 2048, fake(2), fake(2), 16, 2.0, fake(2), None, FAKE, need, None) == \
        q.NF4_ERR_SHAPE
    # the workspace: one byte short is refused, and sizes past the limits give 0
    assert f(2, ptrs(a, b), FAKE, 2048, fake(2), fake(2), 16, 2.0, fake(2), None, FAKE, need - 1, None) == \
        q.NF4_ERR_WORKSPACE
    assert f(2, ptrs(a, b), FAKE, 2048, fake(2), fake(2), 24, 2.0, fake(2), None, FAKE, need, None) == q.NF4_ERR_RANK
    assert q.lib.qlora_workspace_bytes_group(2, (ctypes.c_int64 * 2)(4096, 1000), 2048, 4096, 16) == 0
    assert q.lib.qlora_workspace_bytes_group(0, n2, 2048, 4096, 16) == 0
    # the u of every linear plus at least the group launch's tail: 3 x 1024 tiles... of (4096, 1024, 1024)
    # at 2048 tokens: 48 column tiles x 8 row blocks = 384 tiles, 128 past the first round in 2 ranges
    n3 = (ctypes.c_int64 * 3)(4096, 1024, 1024)
    assert q.lib.qlora_workspace_bytes_group(3, n3, 2048, 4096, 16) >= 3 * 2048 * 16 * 4 + 2 * 128 * 256 * 128 * 4


def test_recompute_validation():
    w = ctypes.byref(_w())
    f = lib.qlora_linear_fwd_recompute
    assert f(w, FAKE, 64, FAKE, FAKE, 16, 2.0, None, FAKE, None, 0, None) == q.NF4_ERR_NULL
    assert f(w, FAKE, 64, FAKE, FAKE, 20, 2.0, FAKE, FAKE, None, 0, None) == q.NF4_ERR_RANK
    assert f(w, FAKE, 64, FAKE, FAKE, 16, 2.0, MISALIGNED, FAKE, None, 0, None) == q.NF4_ERR_ALIGN
    # the skinny path (M <= 16) needs a workspace
    assert f(w, FAKE, 8, FAKE, FAKE, 16, 2.0, FAKE, FAKE, None, 0, None) == q.NF4_ERR_WORKSPACE
    assert f(w, FAKE, 0, FAKE, FAKE, 16, 2.0, FAKE, FAKE, None, 0, None) == q.NF4_OK


def test_bwd_validation():
    w = ctypes.byref(_w())
    ws = q.qlora_workspace_bytes(64, 4096, 4096, 16)
    f = lib.qlora_linear_bwd
    ok = [w, FAKE, FAKE, 64, FAKE, FAKE, 16, 2.0, FAKE, FAKE, FAKE, FAKE, 0, FAKE, ws, None]

    def call(**kw):
        a = list(ok)
        pos = {"x": 1, "dy": 2, "M": 3, "A": 4, "B": 5, "r": 6, "u": 8, "dx": 9, "dA": 10, "dB": 11,
               "ws": 13, "ws_bytes": 14}
        for k, v in kw.items():
            a[pos[k]] = v
        return f(*a)

    assert call(r=48 + 1) == q.NF4_ERR_RANK
    assert call(M=-2) == q.NF4_ERR_SHAPE
    assert call(u=None) == q.NF4_ERR_NULL
    assert call(dA=None) == q.NF4_ERR_NULL
    assert call(dy=MISALIGNED) == q.NF4_ERR_ALIGN
    assert call(ws=None) == q.NF4_ERR_WORKSPACE
    assert call(ws_bytes=ws // 4) == q.NF4_ERR_WORKSPACE
    assert call(M=0) == q.NF4_OK


@pytest.mark.parametrize("M,N,K", [
    (64, 65536, 65536),      # N*K = 2^32: the backward's packed-weight record passes 2^31 bytes
    (64, 1 << 21, 4096),     # N*K = 2^33
    (64, 1 << 22, 64),       # N = 2^22: a 256-row activation tile of dY passes 2^31 bytes
    (64, 16, 1 << 22),       # K = 2^22: the same for x
    (1 << 31, 4096, 4096),   # M = 2^31
    (1 << 30, 16, 1 << 21),  # 2^24 row tiles x 2^14 column tiles: 2^38 workgroups
])
def test_linear_sizes_past_32_bit_offsets_are_refused(M, N, K):
    w = ctypes.byref(_w(N=N, K=K))
    big = 1 << 50   # a workspace size that is never the reason for a refusal
    assert q.qlora_workspace_bytes(M, N, K, 16) == 0
    assert lib.qlora_linear_fwd(w, FAKE, M, FAKE, FAKE, 16, 2.0, FAKE, None, FAKE, big, None) == q.NF4_ERR_SHAPE
    assert lib.qlora_linear_fwd_recompute(w, FAKE, M, FAKE, FAKE, 16, 2.0, FAKE, FAKE, FAKE, big, None) == \
        q.NF4_ERR_SHAPE
    assert lib.qlora_linear_bwd(w, FAKE, FAKE, M, FAKE, FAKE, 16, 2.0, FAKE, FAKE, FAKE, FAKE, 0, FAKE, big,
                                None) == q.NF4_ERR_SHAPE


@pytest.mark.parametrize("M,N,K", [(64, 65536, 65472), (64, (1 << 22) - 16, 1024), (64, 1024, (1 << 22) - 64),
                                   (1 << 20, 4096, 4096)])
def test_linear_sizes_just_inside_the_limits_are_accepted(M, N, K):
    assert q.qlora_workspace_bytes(M, N, K, 16) > 0
    # every argument check passes: only the missing workspace is reported
    w = ctypes.byref(_w(N=N, K=K))
    assert lib.qlora_linear_fwd(w, FAKE, M, FAKE, FAKE, 16, 2.0, FAKE, None, None, 0, None) == q.NF4_ERR_WORKSPACE


def _ptrs(*vals):
    return (ctypes.c_void_p * len(vals))(*vals)


def _numels(*vals):
    return (ctypes.c_int64 * len(vals))(*vals)


def test_adamw_plan_create_validation():
    f = lib.qlora_adamw_plan_create
    l2, n2 = _ptrs(FAKE, FAKE), _numels(4096, 8192)
    out = ctypes.c_void_p(FAKE)

    def call(count=2, params=l2, grads=l2, m=l2, v=l2, pb=None, numel=n2, out_ref=True):
        return f(count, params, grads, m, v, pb, numel, ctypes.byref(out) if out_ref else None)

    assert call(out_ref=False) == q.NF4_ERR_NULL
    assert call(count=0) == q.NF4_ERR_SHAPE
    assert out.value is None                      # cleared on every error
    assert call(numel=None) == q.NF4_ERR_NULL
    assert call(numel=_numels(4096, 10)) == q.NF4_ERR_SHAPE
    assert call(numel=_numels(0, 8)) == q.NF4_ERR_SHAPE
    assert call(numel=_numels(-4, 8)) == q.NF4_ERR_SHAPE
    for key in ("params", "grads", "m", "v"):
        assert call(**{key: None}) == q.NF4_ERR_NULL
        assert call(**{key: _ptrs(FAKE, None)}) == q.NF4_ERR_NULL
        assert call(**{key: _ptrs(MISALIGNED, FAKE)}) == q.NF4_ERR_ALIGN
    assert call(pb=_ptrs(FAKE, FAKE + 2)) == q.NF4_ERR_ALIGN


def test_adamw_plan_step_validation():
    # every check below returns before the plan is dereferenced, so a fake handle is safe
    f = lib.qlora_adamw_plan_step
    good = q.AdamWConfig().c_struct()
    assert f(None, ctypes.byref(good), 1, None, None) == q.NF4_ERR_NULL
    assert f(FAKE, None, 1, None, None) == q.NF4_ERR_NULL
    assert f(FAKE, ctypes.byref(good), 1, FAKE + 4, None) == q.NF4_ERR_ALIGN
    assert f(FAKE, ctypes.byref(good), 0, None, None) == q.NF4_ERR_SHAPE
    for bad in (dict(beta1=1.0), dict(beta2=-0.1), dict(eps=0.0), dict(lr=-1.0),
                dict(weight_decay=-0.5), dict(lr=float("nan")), dict(max_grad_norm=float("inf"))):
        cfg = q.AdamWConfig(**{**q.AdamWConfig().__dict__, **bad}).c_struct()
        assert f(FAKE, ctypes.byref(cfg), 1, None, None) == q.NF4_ERR_SHAPE, bad
    assert lib.qlora_adamw_plan_destroy(None) == q.NF4_OK


def test_q4_codebooks_equal_oracle():
    from oracle import toy
    for book, ref in ((0, oracle.codebook()), (1, toy.fp4_codebook()), (2, toy.int4_codebook())):
        out = (ctypes.c_float * 16)()
        n = lib.q4_codebook_values(book, out)
        assert n == ref.size
        assert np.array_equal(np.array(out[:n], dtype=np.float32), ref)
    assert lib.q4_codebook_values(3, (ctypes.c_float * 16)()) < 0


def test_q4_validation():
    f, g = lib.q4_quantize, lib.q4_dequant
    assert f(FAKE, 4096, 3, 64, FAKE, FAKE, None) == q.NF4_ERR_SHAPE          # codebook
    for bs in (8, 48, 8192):
        assert f(FAKE, 8192, 1, bs, FAKE, FAKE, None) == q.NF4_ERR_SHAPE      # blocksize
    assert f(FAKE, 4096 + 32, 0, 32, FAKE, FAKE, None) == q.NF4_ERR_SHAPE     # numel % 64
    assert f(FAKE, 4096 + 64, 0, 128, FAKE, FAKE, None) == q.NF4_ERR_SHAPE    # numel % blocksize
    assert f(FAKE, -64, 0, 64, FAKE, FAKE, None) == q.NF4_ERR_SHAPE
    assert f(None, 0, 0, 64, None, None, None) == q.NF4_OK                    # empty
    assert f(None, 4096, 0, 64, FAKE, FAKE, None) == q.NF4_ERR_NULL
    assert f(FAKE, 4096, 0, 64, FAKE, MISALIGNED, None) == q.NF4_ERR_ALIGN
    assert g(FAKE, 4096, 2, 16, None, None, None, FAKE, None) == q.NF4_ERR_NULL     # no scales
    assert g(FAKE, 4096, 2, 16, FAKE, FAKE, FAKE, FAKE, None) == q.NF4_ERR_NULL     # both kinds
    assert g(FAKE, 4096, 2, 16, None, FAKE, None, FAKE, None) == q.NF4_ERR_NULL     # half of DQ
    assert g(FAKE, 4096, 2, 16, FAKE, None, None, None, None) == q.NF4_ERR_NULL
    assert g(FAKE, 4096, 2, 16, MISALIGNED, None, None, FAKE, None) == q.NF4_ERR_ALIGN
    assert g(FAKE, 4096, 2, 24, FAKE, None, None, FAKE, None) == q.NF4_ERR_SHAPE
    assert g(None, 0, 1, 4096, None, None, None, None, None) == q.NF4_OK


def test_double_quant_many_validation():
    f = lib.nf4_double_quant_many
    nb = (ctypes.c_int64 * 2)(256, 300)
    ok = _ptrs(FAKE, FAKE)
    assert f(-1, ok, nb, ok, ok, None) == q.NF4_ERR_SHAPE
    assert f(0, None, None, None, None, None) == q.NF4_OK
    assert f(2, None, nb, ok, ok, None) == q.NF4_ERR_NULL
    assert f(2, ok, None, ok, ok, None) == q.NF4_ERR_NULL
    assert f(2, ok, nb, _ptrs(FAKE, None), ok, None) == q.NF4_ERR_NULL
    assert f(2, ok, nb, ok, _ptrs(MISALIGNED, FAKE), None) == q.NF4_ERR_ALIGN
    assert f(2, ok, (ctypes.c_int64 * 2)(256, -64), ok, ok, None) == q.NF4_ERR_SHAPE
    # empty tensors are skipped, whatever their pointers
    assert f(2, _ptrs(None, None), (ctypes.c_int64 * 2)(0, 0), _ptrs(None, None), _ptrs(None, None), None) == q.NF4_OK
