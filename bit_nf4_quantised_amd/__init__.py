"""NF4-quantised QLoRA linear layer on AMD Instinct MI355X (gfx950): Python binding.

A thin ctypes layer over ``libqlora_nf4.so`` (the C ABI in ``include/qlora_nf4.h``). Every function
only checks tensor placement and marshals device pointers, sizes and the current HIP stream; all
computation runs in the library's HIP kernels. PyTorch supplies device memory and streams.

The library must have been built (``python bit_nf4_quantised_amd/build.py``); importing this
package without it raises ImportError, and there is no CPU fallback.

Operations ("QLoRA, explained", pofe.ai): blockwise absmax NF4 quantisation with two indices per
byte, double quantisation of the scales to E4M3, two-level dequantisation to bf16, and the adapted
linear's forward y = x W~^T + s x A^T B^T and backward (dX, dA, dB; no gradient for W), the
adapter merged into the base for serving, and the adapter update of a training step (global
gradient-norm clipping, then AdamW over A and B).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# NF4_LIBRARY names another build of the same library (the host-sanitised one the CPU tests use)
LIB_PATH = os.environ.get("NF4_LIBRARY") or os.path.join(_HERE, "libqlora_nf4.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first with "
        "`python bit_nf4_quantised_amd/build.py` (hipcc, gfx950). There is no CPU fallback.")

lib = ctypes.CDLL(LIB_PATH)

NF4_OK, NF4_ERR_NULL, NF4_ERR_SHAPE, NF4_ERR_ALIGN, NF4_ERR_RANK, NF4_ERR_WORKSPACE, NF4_ERR_HIP = range(7)


class CNF4Weight(ctypes.Structure):
    """Mirror of ``nf4_weight`` in include/qlora_nf4.h."""
    _fields_ = [("packed", ctypes.c_void_p), ("scale_q", ctypes.c_void_p),
                ("scale_c2", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("absmax", ctypes.c_void_p), ("codebook", ctypes.c_int32)]


class CAdamWConfig(ctypes.Structure):
    """Mirror of ``qlora_adamw_config`` in include/qlora_nf4.h."""
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("max_grad_norm", ctypes.c_float)]


_p, _i64, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_W = ctypes.POINTER(CNF4Weight)
_SIGS = {
    "nf4_quantize": (ctypes.c_int, [_p, _i64, _p, _p, _p]),
    "nf4_quantize_bf16": (ctypes.c_int, [_p, _i64, _p, _p, _p]),
    "nf4_double_quant": (ctypes.c_int, [_p, _i64, _p, _p, _p]),
    "nf4_double_quant_many": (ctypes.c_int, [_i64, _p, _p, _p, _p, _p]),
    "nf4_dequant": (ctypes.c_int, [_W, _p, _p]),
    "qlora_linear_fwd": (ctypes.c_int, [_W, _p, _i64, _p, _p, _i32, _f32, _p, _p, _p, _sz, _p]),
    "qlora_linear_fwd_noalloc": (ctypes.c_int, [_W, _p, _i64, _p, _p, _i32, _f32, _p, _p, _p]),
    "qlora_linear_fwd_group": (ctypes.c_int, [_i32, _p, _p, _i64, _p, _p, _i32, _f32, _p, _p, _p, _sz, _p]),
    "qlora_linear_fwd_recompute_group": (ctypes.c_int, [_i32, _p, _p, _i64, _p, _p, _i32, _f32, _p, _p, _p, _sz,
                                                        _p]),
    "qlora_linear_bwd": (ctypes.c_int, [_W, _p, _p, _i64, _p, _p, _i32, _f32, _p, _p, _p, _p,
                                        ctypes.c_int, _p, _sz, _p]),
    "qlora_linear_fwd_recompute": (ctypes.c_int, [_W, _p, _i64, _p, _p, _i32, _f32, _p, _p, _p, _sz,
                                                  _p]),
    "qlora_merge": (ctypes.c_int, [_W, _p, _p, _i32, _f32, _p, _p]),
    "q4_codebook_values": (ctypes.c_int, [_i32, ctypes.POINTER(ctypes.c_float)]),
    "q4_quantize": (ctypes.c_int, [_p, _i64, _i32, _i32, _p, _p, _p]),
    "q4_dequant": (ctypes.c_int, [_p, _i64, _i32, _i32, _p, _p, _p, _p, _p]),
    "qlora_adamw_plan_create": (ctypes.c_int, [_i64, _p, _p, _p, _p, _p, _p,
                                               ctypes.POINTER(ctypes.c_void_p)]),
    "qlora_adamw_plan_step": (ctypes.c_int, [_p, ctypes.POINTER(CAdamWConfig), _i64, _p, _p]),
    "qlora_adamw_plan_destroy": (ctypes.c_int, [_p]),
    "qlora_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "qlora_workspace_bytes_group": (_sz, [_i32, _p, _i64, _i64, _i32]),
    "qlora_linear_bwd_group": (ctypes.c_int, [_i32, _p, _p, _p, _i64, _p, _p, _i32, _f32, _p, _p, _p, _p,
                                              ctypes.c_int, _p, _sz, _p]),
    "nf4_storage_bytes": (_i64, [_i64]),
    "nf4_codebook": (None, [ctypes.POINTER(ctypes.c_float)]),
    "nf4_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


class NF4Error(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {lib.nf4_status_string(status).decode()} (status {status})")


def _check(status: int, call: str) -> None:
    if status != NF4_OK:
        raise NF4Error(status, call)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dtype(t, *allowed):
    if t is not None and t.dtype not in allowed:
        raise TypeError(f"dtype {t.dtype} not in {allowed}")


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


@dataclass
class NF4Weight:
    """A quantised N x K weight in device tensors: double-quantised scales (scale_q, scale_c2) or,
    without double quantisation, the fp32 absmax (scale_q and scale_c2 None). codebook: the values
    the indices select (0 NF4, 1 FP4, 2 INT4; see Q4_CODEBOOKS)."""
    packed: torch.Tensor           # uint8 [N*K/2]
    scale_q: torch.Tensor | None   # uint8 [N*K/64]
    scale_c2: torch.Tensor | None  # float32 [ceil(N*K/16384)]
    N: int
    K: int
    absmax: torch.Tensor | None = None   # float32 [N*K/64]
    codebook: int = 0

    def c_struct(self) -> CNF4Weight:
        return CNF4Weight(_ptr(self.packed), _ptr(self.scale_q), _ptr(self.scale_c2), self.N, self.K,
                          _ptr(self.absmax), _book(self.codebook))


# ------------------------------------------------------------------------- the five calls
def nf4_quantize(w, packed, absmax, stream=None) -> None:
    _dtype(w, torch.float32); _dtype(packed, torch.uint8); _dtype(absmax, torch.float32)
    n = w.numel()
    if packed.numel() * 2 != n or absmax.numel() * 64 != n:
        raise ValueError("output sizes must be numel/2 and numel/64")
    _check(lib.nf4_quantize(_ptr(w), n, _ptr(packed), _ptr(absmax), _stream(stream)), "nf4_quantize")


def nf4_quantize_bf16(w, packed, absmax, stream=None) -> None:
    """nf4_quantize of a bf16 array (a merged weight quantised again)."""
    _dtype(w, *_BF16); _dtype(packed, torch.uint8); _dtype(absmax, torch.float32)
    n = w.numel()
    if packed.numel() * 2 != n or absmax.numel() * 64 != n:
        raise ValueError("output sizes must be numel/2 and numel/64")
    _check(lib.nf4_quantize_bf16(_ptr(w), n, _ptr(packed), _ptr(absmax), _stream(stream)),
           "nf4_quantize_bf16")


def nf4_double_quant(absmax, scale_q, scale_c2, stream=None) -> None:
    _dtype(absmax, torch.float32); _dtype(scale_q, torch.uint8); _dtype(scale_c2, torch.float32)
    nb = absmax.numel()
    if scale_q.numel() != nb or scale_c2.numel() != (nb + 255) // 256:
        raise ValueError("output sizes must be nblocks and ceil(nblocks/256)")
    _check(lib.nf4_double_quant(_ptr(absmax), nb, _ptr(scale_q), _ptr(scale_c2), _stream(stream)),
           "nf4_double_quant")


class DoubleQuantMany:
    """nf4_double_quant_many over fixed lists of tensors, with the argument arrays marshalled once
    (a model's weights at load time); calling it enqueues the launches on the stream."""

    def __init__(self, absmax: list, scale_q: list, scale_c2: list):
        n = len(absmax)
        if len(scale_q) != n or len(scale_c2) != n:
            raise ValueError("one scale_q and scale_c2 per absmax")
        for a, c, g in zip(absmax, scale_q, scale_c2):
            _dtype(a, torch.float32); _dtype(c, torch.uint8); _dtype(g, torch.float32)
            if c.numel() != a.numel() or g.numel() != (a.numel() + 255) // 256:
                raise ValueError("output sizes must be nblocks and ceil(nblocks/256)")
        P = ctypes.c_void_p * max(n, 1)
        self._keep = (list(absmax), list(scale_q), list(scale_c2))   # the tensors stay alive
        self._args = (n, P(*[_ptr(a) for a in absmax]), (ctypes.c_int64 * max(n, 1))(*[a.numel() for a in absmax]),
                      P(*[_ptr(c) for c in scale_q]), P(*[_ptr(g) for g in scale_c2]))

    def __call__(self, stream=None) -> None:
        _check(lib.nf4_double_quant_many(*self._args, _stream(stream)), "nf4_double_quant_many")


def nf4_double_quant_many(absmax: list, scale_q: list, scale_c2: list, stream=None) -> None:
    """nf4_double_quant over several weights' scales (up to 64 per kernel launch)."""
    DoubleQuantMany(absmax, scale_q, scale_c2)(stream)


def nf4_dequant(weight: NF4Weight, out, stream=None) -> None:
    _dtype(out, *_BF16)
    if out.numel() != weight.N * weight.K:
        raise ValueError("out must hold N*K values")
    cw = weight.c_struct()
    _check(lib.nf4_dequant(ctypes.byref(cw), _ptr(out), _stream(stream)), "nf4_dequant")


def qlora_linear_fwd(weight: NF4Weight, x, A, B, scale: float, y, u_out=None, ws=None,
                     stream=None) -> None:
    for t in (x, A, B, y):
        _dtype(t, *_BF16)
    _dtype(u_out, torch.float32)
    M = x.shape[0]
    r = A.shape[0]
    if x.shape != (M, weight.K) or A.shape != (r, weight.K) or B.shape != (weight.N, r) \
            or y.shape != (M, weight.N) or (u_out is not None and u_out.numel() != M * r):
        raise ValueError("shape mismatch")
    if ws is None:
        ws = workspace(M, weight.N, weight.K, r, x.device)
    cw = weight.c_struct()
    _check(lib.qlora_linear_fwd(ctypes.byref(cw), _ptr(x), M, _ptr(A), _ptr(B), r, scale, _ptr(y),
                                _ptr(u_out), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream)), "qlora_linear_fwd")


def qlora_workspace_bytes_group(M: int, N: list, K: int, r: int) -> int:
    n = (ctypes.c_int64 * max(len(N), 1))(*[int(v) for v in N])
    return int(lib.qlora_workspace_bytes_group(len(N), n, M, K, r))


def workspace_group(M: int, N: list, K: int, r: int, device="cuda") -> torch.Tensor:
    """A device workspace large enough for qlora_linear_fwd_group over weights of N rows."""
    nbytes = max(qlora_workspace_bytes_group(M, N, K, r), 256)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def qlora_linear_fwd_group(weights: list, x, As: list, Bs: list, scale: float, ys: list, us=None, ws=None,
                           stream=None) -> None:
    """Forward of several linears that share x (e.g. q/k/v or gate/up): ys[i] = x W~_i^T +
    s (x A_i^T) B_i^T, as one fused launch where the shapes allow (see qlora_linear_fwd_group in
    include/qlora_nf4.h); us[i] (optional) receives u_i = x A_i^T."""
    n = len(weights)
    if not (len(As) == len(Bs) == len(ys) == n) or (us is not None and len(us) != n):
        raise ValueError("one A, B and y (and u) per weight")
    _dtype(x, *_BF16)
    M = x.shape[0]
    r = As[0].shape[0]
    for w, A, B, y in zip(weights, As, Bs, ys):
        for t in (A, B, y):
            _dtype(t, *_BF16)
        if x.shape != (M, w.K) or A.shape != (r, w.K) or B.shape != (w.N, r) or y.shape != (M, w.N):
            raise ValueError("shape mismatch")
    if us is not None:
        for u in us:
            _dtype(u, torch.float32)
            if u is not None and u.numel() != M * r:
                raise ValueError("shape mismatch")
    if ws is None:
        ws = workspace_group(M, [w.N for w in weights], weights[0].K, r, x.device)
    cws = [w.c_struct() for w in weights]
    P = ctypes.c_void_p
    wp = (P * n)(*[ctypes.addressof(c) for c in cws])
    ap = (P * n)(*[_ptr(A) for A in As])
    bp = (P * n)(*[_ptr(B) for B in Bs])
    yp = (P * n)(*[_ptr(y) for y in ys])
    up = (P * n)(*[_ptr(u) for u in us]) if us is not None else None
    _check(lib.qlora_linear_fwd_group(n, wp, _ptr(x), M, ap, bp, r, scale, yp, up, _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)), "qlora_linear_fwd_group")


def qlora_linear_fwd_recompute_group(weights: list, x, As: list, Bs: list, scale: float, us: list, ys: list,
                                     ws=None, stream=None) -> None:
    """qlora_linear_fwd_group with every u_i = x A_i^T known: the fused GEMMs only."""
    n = len(weights)
    if not (len(As) == len(Bs) == len(ys) == len(us) == n):
        raise ValueError("one A, B, u and y per weight")
    _dtype(x, *_BF16)
    M = x.shape[0]
    r = As[0].shape[0]
    for w, A, B, y, u in zip(weights, As, Bs, ys, us):
        for t in (A, B, y):
            _dtype(t, *_BF16)
        _dtype(u, torch.float32)
        if x.shape != (M, w.K) or A.shape != (r, w.K) or B.shape != (w.N, r) or y.shape != (M, w.N) \
                or u.numel() != M * r:
            raise ValueError("shape mismatch")
    if ws is None:
        ws = workspace_group(M, [w.N for w in weights], weights[0].K, r, x.device)
    cws = [w.c_struct() for w in weights]
    P = ctypes.c_void_p
    wp = (P * n)(*[ctypes.addressof(c) for c in cws])
    _check(lib.qlora_linear_fwd_recompute_group(n, wp, _ptr(x), M, (P * n)(*[_ptr(A) for A in As]),
                                                (P * n)(*[_ptr(B) for B in Bs]), r, scale,
                                                (P * n)(*[_ptr(u) for u in us]), (P * n)(*[_ptr(y) for y in ys]),
                                                _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "qlora_linear_fwd_recompute_group")


def qlora_linear_bwd_group(weights: list, x, dys: list, As: list, Bs: list, scale: float, us: list, dxs,
                           dAs: list, dBs: list, accumulate: bool = False, ws=None, stream=None) -> None:
    """Backward of several linears that share x: for each i as qlora_linear_bwd (dxs[i], dAs[i],
    dBs[i]), the dX GEMMs as one launch where the shapes allow; dxs None skips the input gradients."""
    n = len(weights)
    if not (len(dys) == len(As) == len(Bs) == len(us) == len(dAs) == len(dBs) == n) or \
            (dxs is not None and len(dxs) != n):
        raise ValueError("one dY, A, B, u, dA and dB (and dX) per weight")
    _dtype(x, *_BF16)
    M = x.shape[0]
    r = As[0].shape[0]
    for i, w in enumerate(weights):
        for t in (dys[i], As[i], Bs[i]) + ((dxs[i],) if dxs is not None else ()):
            _dtype(t, *_BF16)
        for t in (us[i], dAs[i], dBs[i]):
            _dtype(t, torch.float32)
        if x.shape != (M, w.K) or dys[i].shape != (M, w.N) or As[i].shape != (r, w.K) or Bs[i].shape != (w.N, r) \
                or us[i].numel() != M * r or dAs[i].shape != (r, w.K) or dBs[i].shape != (w.N, r) \
                or (dxs is not None and dxs[i].shape != (M, w.K)):
            raise ValueError("shape mismatch")
    if ws is None:
        ws = workspace_group(M, [w.N for w in weights], weights[0].K, r, x.device)
    cws = [w.c_struct() for w in weights]
    P = ctypes.c_void_p
    arr = lambda ts: (P * n)(*[_ptr(t) for t in ts])  # noqa: E731
    _check(lib.qlora_linear_bwd_group(n, (P * n)(*[ctypes.addressof(c) for c in cws]), _ptr(x), arr(dys), M,
                                      arr(As), arr(Bs), r, scale, arr(us), arr(dxs) if dxs is not None else None,
                                      arr(dAs), arr(dBs), int(bool(accumulate)), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)), "qlora_linear_bwd_group")


def qlora_linear_fwd_noalloc(weight: NF4Weight, x, A, B, scale: float, y, u_out=None,
                             stream=None) -> None:
    """qlora_linear_fwd with the library's own per-GPU workspace (no allocation anywhere)."""
    for t in (x, A, B, y):
        _dtype(t, *_BF16)
    _dtype(u_out, torch.float32)
    M = x.shape[0]
    r = A.shape[0]
    if x.shape != (M, weight.K) or A.shape != (r, weight.K) or B.shape != (weight.N, r) \
            or y.shape != (M, weight.N) or (u_out is not None and u_out.numel() != M * r):
        raise ValueError("shape mismatch")
    cw = weight.c_struct()
    _check(lib.qlora_linear_fwd_noalloc(ctypes.byref(cw), _ptr(x), M, _ptr(A), _ptr(B), r, scale, _ptr(y),
                                        _ptr(u_out), _stream(stream)), "qlora_linear_fwd_noalloc")


def qlora_merge(weight: NF4Weight, A, B, scale: float, out, stream=None) -> None:
    """Adapter merged into the dequantised base: out = bf16(W~ + s B A), [N x K]."""
    for t in (A, B, out):
        _dtype(t, *_BF16)
    r = A.shape[0]
    if A.shape != (r, weight.K) or B.shape != (weight.N, r) or out.numel() != weight.N * weight.K:
        raise ValueError("shape mismatch")
    cw = weight.c_struct()
    _check(lib.qlora_merge(ctypes.byref(cw), _ptr(A), _ptr(B), r, scale, _ptr(out), _stream(stream)),
           "qlora_merge")


def qlora_linear_fwd_recompute(weight: NF4Weight, x, A, B, scale: float, u, y, ws=None,
                               stream=None) -> None:
    """Forward with a known u = x A^T (gradient-checkpointing recompute): the forward's GEMM
    without the pass that forms u."""
    for t in (x, A, B, y):
        _dtype(t, *_BF16)
    _dtype(u, torch.float32)
    M = x.shape[0]
    r = A.shape[0]
    if x.shape != (M, weight.K) or A.shape != (r, weight.K) or B.shape != (weight.N, r) \
            or y.shape != (M, weight.N) or u.numel() != M * r:
        raise ValueError("shape mismatch")
    if ws is None:   # with the forward's workspace the launches (and y) are the forward's own
        ws = workspace(M, weight.N, weight.K, r, x.device)
    cw = weight.c_struct()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.qlora_linear_fwd_recompute(ctypes.byref(cw), _ptr(x), M, _ptr(A), _ptr(B), r, scale,
                                          _ptr(u), _ptr(y), _ptr(ws), nbytes, _stream(stream)),
           "qlora_linear_fwd_recompute")


def qlora_linear_bwd(weight: NF4Weight, x, dy, A, B, scale: float, u, dx, dA, dB,
                     accumulate: bool = False, ws=None, stream=None) -> None:
    for t in (x, dy, A, B, dx):
        _dtype(t, *_BF16)
    for t in (u, dA, dB):
        _dtype(t, torch.float32)
    M = x.shape[0]
    r = A.shape[0]
    if x.shape != (M, weight.K) or dy.shape != (M, weight.N) or A.shape != (r, weight.K) \
            or B.shape != (weight.N, r) or u.numel() != M * r or dA.shape != (r, weight.K) \
            or dB.shape != (weight.N, r) or (dx is not None and dx.shape != (M, weight.K)):
        raise ValueError("shape mismatch")
    if ws is None:
        ws = workspace(M, weight.N, weight.K, r, x.device)
    cw = weight.c_struct()
    _check(lib.qlora_linear_bwd(ctypes.byref(cw), _ptr(x), _ptr(dy), M, _ptr(A), _ptr(B), r, scale,
                                _ptr(u), _ptr(dx), _ptr(dA), _ptr(dB), int(bool(accumulate)),
                                _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "qlora_linear_bwd")


# ------------------------------------------------------------------------- format variants
Q4_CODEBOOKS = {"nf4": 0, "fp4": 1, "int4": 2}


def _book(codebook) -> int:
    if isinstance(codebook, str):
        if codebook not in Q4_CODEBOOKS:
            raise ValueError(f"codebook must be one of {sorted(Q4_CODEBOOKS)}")
        return Q4_CODEBOOKS[codebook]
    return int(codebook)


def q4_codebook_values(codebook) -> list:
    out = (ctypes.c_float * 16)()
    n = lib.q4_codebook_values(_book(codebook), out)
    if n < 0:
        raise NF4Error(-n, "q4_codebook_values")
    return list(out)[:n]


def q4_quantize(w, codebook, blocksize: int, packed, absmax, stream=None) -> None:
    """Blockwise absmax quantisation with the NF4, FP4 or INT4 codebook and blocksize 16..4096."""
    _dtype(w, torch.float32); _dtype(packed, torch.uint8); _dtype(absmax, torch.float32)
    n = w.numel()
    if packed.numel() * 2 != n or absmax.numel() * blocksize != n:
        raise ValueError("output sizes must be numel/2 and numel/blocksize")
    _check(lib.q4_quantize(_ptr(w), n, _book(codebook), blocksize, _ptr(packed), _ptr(absmax),
                           _stream(stream)), "q4_quantize")


def q4_dequant(packed, numel: int, codebook, blocksize: int, out, absmax=None, scale_q=None,
               scale_c2=None, stream=None) -> None:
    """bf16 weights from packed indices and either fp32 scales (absmax) or double-quantised ones
    (scale_q, scale_c2)."""
    _dtype(packed, torch.uint8); _dtype(out, *_BF16); _dtype(absmax, torch.float32)
    _dtype(scale_q, torch.uint8); _dtype(scale_c2, torch.float32)
    if packed.numel() * 2 != numel or out.numel() != numel:
        raise ValueError("packed must hold numel/2 bytes and out numel values")
    nb = numel // blocksize
    if (absmax is not None and absmax.numel() != nb) or (scale_q is not None and scale_q.numel() != nb) \
            or (scale_c2 is not None and scale_c2.numel() != (nb + 255) // 256):
        raise ValueError("scale sizes do not match numel / blocksize")
    _check(lib.q4_dequant(_ptr(packed), numel, _book(codebook), blocksize, _ptr(absmax), _ptr(scale_q),
                          _ptr(scale_c2), _ptr(out), _stream(stream)), "q4_dequant")


# ------------------------------------------------------------------------- the adapter update
@dataclass(frozen=True)
class AdamWConfig:
    """Hyper-parameters of the adapter update; lr and the clipping threshold are the ones "QLoRA,
    explained" gives (The algorithm, step by step; Minimal implementation), the rest torch's AdamW
    defaults."""
    lr: float = 2e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    max_grad_norm: float = 0.3   # <= 0: no clipping

    def c_struct(self) -> CAdamWConfig:
        return CAdamWConfig(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay,
                            self.max_grad_norm)


def _ptr_array(tensors, dtypes, allow_none=False):
    arr = (ctypes.c_void_p * len(tensors))()
    for i, t in enumerate(tensors):
        if t is None and allow_none:
            arr[i] = None
            continue
        _dtype(t, *dtypes)
        arr[i] = _ptr(t)
    return arr


class AdamWPlan:
    """qlora_adamw_plan over a set of adapter tensors (fp32 master weights, gradients, first and
    second moments, optional bf16 copies): one call runs the clipped AdamW step over all of them
    in three kernel launches. The tensors must stay alive, at the same storage, while the plan is
    used; the plan keeps references to them."""

    def __init__(self, params, grads, exp_avg, exp_avg_sq, params_bf16=None,
                 cfg: AdamWConfig = AdamWConfig()):
        n = len(params)
        if not (len(grads) == len(exp_avg) == len(exp_avg_sq) == n) or n == 0 or \
                (params_bf16 is not None and len(params_bf16) != n):
            raise ValueError("tensor lists differ in length or are empty")
        for i in range(n):
            sizes = [grads[i].numel(), exp_avg[i].numel(), exp_avg_sq[i].numel()]
            if params_bf16 is not None and params_bf16[i] is not None:
                sizes.append(params_bf16[i].numel())
            if any(k != params[i].numel() for k in sizes):
                raise ValueError(f"tensor {i}: sizes differ")
        self._keep = (list(params), list(grads), list(exp_avg), list(exp_avg_sq),
                      None if params_bf16 is None else list(params_bf16))
        self.cfg = cfg
        self._ccfg = cfg.c_struct()
        f32 = (torch.float32,)
        pb = None if params_bf16 is None else _ptr_array(params_bf16, _BF16, allow_none=True)
        numel = (ctypes.c_int64 * n)(*[t.numel() for t in params])
        handle = ctypes.c_void_p()
        with torch.cuda.device(params[0].device):
            _check(lib.qlora_adamw_plan_create(n, _ptr_array(params, f32), _ptr_array(grads, f32),
                                               _ptr_array(exp_avg, f32), _ptr_array(exp_avg_sq, f32),
                                               pb, numel, ctypes.byref(handle)),
                   "qlora_adamw_plan_create")
        self._handle = handle
        self.values = sum(t.numel() for t in params)

    def step(self, step: int, grad_norm=None, stream=None) -> None:
        """AdamW step number `step` (from 1); grad_norm (one float64 on the device) receives the
        gradient norm before clipping."""
        _dtype(grad_norm, torch.float64)
        _check(lib.qlora_adamw_plan_step(self._handle, ctypes.byref(self._ccfg), int(step),
                                         _ptr(grad_norm), _stream(stream)), "qlora_adamw_plan_step")

    def close(self) -> None:
        if getattr(self, "_handle", None) is not None and self._handle.value:
            lib.qlora_adamw_plan_destroy(self._handle)
        self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover - interpreter shutdown
            pass


# ------------------------------------------------------------------------- helpers
def qlora_workspace_bytes(M: int, N: int, K: int, r: int) -> int:
    return int(lib.qlora_workspace_bytes(M, N, K, r))


def nf4_storage_bytes(numel: int) -> int:
    return int(lib.nf4_storage_bytes(numel))


def nf4_codebook() -> list:
    out = (ctypes.c_float * 16)()
    lib.nf4_codebook(out)
    return list(out)


def workspace(M: int, N: int, K: int, r: int, device="cuda") -> torch.Tensor:
    """A device workspace large enough for qlora_linear_fwd/bwd at these sizes."""
    nbytes = max(qlora_workspace_bytes(M, N, K, r), 256)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def empty_weight(N: int, K: int, device="cuda", codebook=0) -> NF4Weight:
    nb = N * K // 64
    return NF4Weight(torch.empty(N * K // 2, dtype=torch.uint8, device=device),
                     torch.empty(nb, dtype=torch.uint8, device=device),
                     torch.empty((nb + 255) // 256, dtype=torch.float32, device=device), N, K,
                     codebook=_book(codebook))


def quantize_weight(w: torch.Tensor, stream=None, absmax: torch.Tensor | None = None,
                    double_quant: bool = True, codebook=0) -> NF4Weight:
    """Quantise a float32 N x K device tensor: nf4_quantize (q4_quantize at blocksize 64 for the FP4
    or INT4 codebook) followed by nf4_double_quant, or with double_quant=False a weight that keeps
    the fp32 absmax as its scales."""
    N, K = w.shape
    book = _book(codebook)
    if absmax is None:
        absmax = torch.empty(N * K // 64, dtype=torch.float32, device=w.device)
    if not double_quant:
        qw = NF4Weight(torch.empty(N * K // 2, dtype=torch.uint8, device=w.device), None, None, N, K, absmax,
                       codebook=book)
    else:
        qw = empty_weight(N, K, w.device, book)
    if book == 0:
        nf4_quantize(w, qw.packed, absmax, stream)
    else:
        q4_quantize(w, book, 64, qw.packed, absmax, stream)
    if double_quant:
        nf4_double_quant(absmax, qw.scale_q, qw.scale_c2, stream)
    return qw


__all__ = ["lib", "LIB_PATH", "EXPORTED", "NF4Error", "NF4Weight", "CNF4Weight", "nf4_quantize",
           "nf4_quantize_bf16",
           "nf4_double_quant", "nf4_double_quant_many", "DoubleQuantMany", "nf4_dequant", "qlora_linear_fwd", "qlora_linear_fwd_noalloc",
           "qlora_linear_fwd_recompute", "qlora_linear_fwd_group", "qlora_linear_fwd_recompute_group",
           "qlora_workspace_bytes_group", "qlora_linear_bwd_group",
           "workspace_group",
           "qlora_linear_bwd", "qlora_merge", "AdamWConfig", "CAdamWConfig", "AdamWPlan",
           "Q4_CODEBOOKS", "q4_codebook_values", "q4_quantize", "q4_dequant",
           "qlora_workspace_bytes", "nf4_storage_bytes", "nf4_codebook", "workspace",
           "empty_weight", "quantize_weight"]
