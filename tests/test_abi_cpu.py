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
    blocks and 2048-column steps with one u partial per activation dword (4 per split), larger M
    256-row blocks and 512-column steps with one u partial per wave (16 per split); the row blocks
    times the k splits fill 256 workgroups at most, and u plus the partials come first."""
    rows, step, uper = (64, 2048, 4) if M <= 4 else (256, 512, 16)
    nsteps = -(-K // step)
    blocks = max(-(-N // rows), r // 16)
    want = min(max(256 // blocks, 1), nsteps)
    sub = -(-nsteps // want)
    splits = -(-nsteps // sub)
    part = ((splits * M * N + 3) // 4) * 4 + splits * uper * M * r
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
