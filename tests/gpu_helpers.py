"""Shared helpers for the GPU parity tests: move seeded inputs to the device, run the library's
calls through the Python binding (which goes through the C ABI), and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

TOL_REL_FRO = 5e-3     # relative Frobenius error bound on GEMM outputs and gradients
TOL_MAX_REL = 1e-2     # elementwise |err| <= 1e-2 * max |ref|


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(dev())


def bf16_to_dev(bits: np.ndarray) -> torch.Tensor:
    return to_dev(bits.view(np.int16))


def bits_from_dev(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def f64_from_bits(bits: np.ndarray) -> np.ndarray:
    return oracle.f32_from_bf16_bits(bits).astype(np.float64)


def assert_close(name: str, got: np.ndarray, ref: np.ndarray) -> None:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    nref = np.linalg.norm(ref)
    err = np.linalg.norm(got - ref)
    rel = err / nref if nref > 0 else err
    mref = np.abs(ref).max() if ref.size else 0.0
    mx = np.abs(got - ref).max() if ref.size else 0.0
    ok = rel <= TOL_REL_FRO and mx <= TOL_MAX_REL * mref + (0.0 if mref > 0 else 1e-30)
    assert ok, f"{name}: rel_fro={rel:.3e} max_err={mx:.3e} max_ref={mref:.3e}"


def gpu_quantize(w: np.ndarray):
    """nf4_quantize + nf4_double_quant on the GPU. Returns (weight, packed, absmax, codes, c2)."""
    import bit_nf4_quantised_amd as q
    N, K = w.shape
    wd = to_dev(w.astype(np.float32))
    absmax = torch.empty(N * K // 64, dtype=torch.float32, device=dev())
    qw = q.quantize_weight(wd, absmax=absmax)
    torch.cuda.synchronize()
    return (qw, qw.packed.cpu().numpy(), absmax.cpu().numpy(), qw.scale_q.cpu().numpy(),
            qw.scale_c2.cpu().numpy())


def gpu_dequant(qw) -> np.ndarray:
    import bit_nf4_quantised_amd as q
    out = torch.empty(qw.N * qw.K, dtype=torch.int16, device=dev())
    q.nf4_dequant(qw, out)
    torch.cuda.synchronize()
    return bits_from_dev(out)


def gpu_fwd_bwd(qw, x, a, b, dy, scale, with_dx=True, accumulate=False, dA0=None, dB0=None):
    """Forward then backward through the binding. Inputs are bf16 bit arrays; returns numpy
    (y bits, u, dx bits or None, dA, dB)."""
    import bit_nf4_quantised_amd as q
    M, K = x.shape
    N = qw.N
    r = a.shape[0]
    X, A, B, DY = bf16_to_dev(x), bf16_to_dev(a), bf16_to_dev(b), bf16_to_dev(dy)
    y = torch.empty(M, N, dtype=torch.int16, device=dev())
    u = torch.empty(M, r, dtype=torch.float32, device=dev())
    ws = q.workspace(M, N, K, r)
    q.qlora_linear_fwd(qw, X, A, B, scale, y, u, ws=ws)
    dx = torch.empty(M, K, dtype=torch.int16, device=dev()) if with_dx else None
    dA = to_dev(dA0) if dA0 is not None else torch.empty(r, K, dtype=torch.float32, device=dev())
    dB = to_dev(dB0) if dB0 is not None else torch.empty(N, r, dtype=torch.float32, device=dev())
    q.qlora_linear_bwd(qw, X, DY, A, B, scale, u, dx, dA, dB, accumulate=accumulate, ws=ws)
    torch.cuda.synchronize()
    return (bits_from_dev(y), u.cpu().numpy(), bits_from_dev(dx) if with_dx else None,
            dA.cpu().numpy(), dB.cpu().numpy())


def oracle_weight(w: np.ndarray) -> np.ndarray:
    """The oracle's dequantised bf16 weight (bits, N x K)."""
    N, K = w.shape
    packed, c1 = oracle.quantize(w)
    codes, c2 = oracle.double_quant(c1)
    return oracle.dequant(packed, codes, c2, N * K).reshape(N, K)
