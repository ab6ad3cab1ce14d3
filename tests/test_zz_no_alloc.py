"""The forward without a workspace argument, called through the C ABI, against qlora_linear_fwd with
a caller-owned workspace: the same launches, so the same outputs bit for bit. Two calls in a row
share the library's per-GPU array; the second is smaller and keeps u in that array."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import assert_close, bf16_to_dev, bits_from_dev, dev, f64_from_bits, gpu_quantize, log, \
    oracle_weight

pytestmark = pytest.mark.gpu


def _inputs(seed, M, N, K, r):
    w = wl.weight("single", 600 + seed, N, K, "gauss", 0.02)
    g = wl.rng_for("single", 600 + seed, "x")
    x = wl.to_bf16_bits(g.standard_normal((M, K), dtype=np.float32))
    a = wl.to_bf16_bits(g.standard_normal((r, K), dtype=np.float32) * np.float32(0.01))
    b = wl.to_bf16_bits(g.standard_normal((N, r), dtype=np.float32) * np.float32(0.01))
    return w, x, a, b


def _compare(M, N, K, r, s, keep_u):
    import bit_nf4_quantised_amd as q
    log(f"[noalloc] M={M} N={N} K={K} r={r} s={s} u_out={'yes' if keep_u else 'NULL'}")
    w, x, a, b = _inputs(M + N + r, M, N, K, r)
    qw = gpu_quantize(w)[0]
    X, A, B = bf16_to_dev(x), bf16_to_dev(a), bf16_to_dev(b)
    y_ref = torch.empty(M, N, dtype=torch.int16, device=dev())
    u_ref = torch.empty(M, r, dtype=torch.float32, device=dev())
    q.qlora_linear_fwd(qw, X, A, B, s, y_ref, u_ref)
    y = torch.full((M, N), -1, dtype=torch.int16, device=dev())
    u = torch.full((M, r), float("nan"), dtype=torch.float32, device=dev()) if keep_u else None
    cw = qw.c_struct()
    st = q.lib.qlora_linear_fwd_noalloc(ctypes.byref(cw), X.data_ptr(), M, A.data_ptr(), B.data_ptr(), r, s,
                                        y.data_ptr(), u.data_ptr() if keep_u else None,
                                        torch.cuda.current_stream().cuda_stream)
    assert st == q.NF4_OK, q.lib.nf4_status_string(st)
    torch.cuda.synchronize()
    assert np.array_equal(bits_from_dev(y), bits_from_dev(y_ref)), "y differs from qlora_linear_fwd"
    if keep_u:
        assert np.array_equal(u.cpu().numpy().view(np.uint32), u_ref.cpu().numpy().view(np.uint32))
    # and the oracle's tolerance, as for every forward
    yr, _ = oracle.linear_fwd(x, oracle_weight(w), a, b, s)
    assert_close("y", f64_from_bits(bits_from_dev(y)), yr)


def test_noalloc_forward_equals_the_workspace_forward_on_consecutive_calls():
    # first: the fused GEMM with its contraction split in two (partial sums in the array)
    _compare(300, 1040, 1088, 48, 0.5, keep_u=True)
    # then smaller: the few-token path (split partials and u, with u_out NULL, in the same array)
    _compare(3, 400, 960, 16, 2.0, keep_u=False)


def test_noalloc_forward_refuses_a_workspace_past_the_array():
    import bit_nf4_quantised_amd as q
    # 16 tokens of a 2^21 x 64 weight: 128 MiB of split partials, past the 64 MiB array
    cw = q.CNF4Weight(0x100000, 0x100000, 0x100000, 1 << 21, 64)
    st = q.lib.qlora_linear_fwd_noalloc(ctypes.byref(cw), 0x100000, 16, 0x100000, 0x100000, 16, 1.0, 0x100000,
                                        None, None)
    assert st == q.NF4_ERR_WORKSPACE
