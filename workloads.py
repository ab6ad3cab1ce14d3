"""Seeded synthetic inputs for the NF4 QLoRA linear layer: shapes and value distributions only.

This module holds none of the method's arithmetic. It draws weights, activations, adapters and
upstream gradients with numpy from a keyed ``SeedSequence(0)`` tree, and rounds the bf16 tensors
with torch's own float32 -> bfloat16 cast, so the CPU oracle and the GPU path see the same bits.
Both the tests and ``bench.py`` import it; neither side of the parity check owns it.

Workloads (sizes as out x in, i.e. W is N x K row-major like ``nn.Linear``):

* ``single``    one 4096 x 4096 linear, 16 tokens, rank 16, alpha 32.
* ``llama8b``   the seven linears of a Llama-3.1-8B layer (q/o 4096x4096, k/v 1024x4096,
                gate/up 14336x4096, down 4096x14336), 2048 tokens, rank 16, alpha 32.
* ``llama65b``  the seven linears of a 65B-shaped layer (q/k/v/o 8192x8192, gate/up 22016x8192,
                down 8192x22016), weights 0.015*N(0,1) with 0.1% of entries scaled by 20,
                4096 tokens, rank 64, alpha 16.
* ``stream``    bandwidth paths: 4096 x 14336 matrices of 0.02*N(0,1) (quantise / double-quantise /
                dequantise), and an 8192 x 28672 weight for the skinny forward at 1, 4 and 16 tokens.
* ``llama70b``  the seven linears of a 70B-shaped block (q/o 8192x8192, k/v 1024x8192,
                gate/up 28672x8192, down 8192x28672), weights 0.015 * t_4 / sqrt(2) (Student-t with
                four degrees of freedom scaled to unit variance), 4096 tokens, rank 64, alpha 16.

Adapters A (r x K) and B (N x r) are N(0, 0.01^2); activations X (M x K) and upstream gradients
dY (M x N) are N(0, 1); all four are rounded to bf16.

The adapter update draws fp32 master copies of A and B, N(0, 0.01^2), for every linear of
``layers`` layers (Llama-3.1-8B: 32 layers, 448 tensors, 41.9 M values at rank 16), and fresh
N(0, sigma^2) fp32 gradients per step (sigma 1e-3 puts the global norm above the 0.3 threshold).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

WORKLOAD_IDS = {"single": 1, "llama8b": 2, "llama65b": 3, "stream": 4, "llama70b": 5}
TENSOR_IDS = {"w": 0, "x": 1, "a": 2, "b": 3, "dy": 4, "grad": 5, "master": 6}


@dataclass(frozen=True)
class Linear:
    name: str
    n: int  # out features
    k: int  # in features


@dataclass(frozen=True)
class Workload:
    name: str
    linears: tuple
    m: int          # tokens
    r: int          # LoRA rank
    alpha: float
    weight_kind: str  # "gauss", "gauss_outlier", "student_t4"
    sigma: float

    @property
    def scale(self) -> float:
        return self.alpha / self.r


def _llama_layer(h, kv, ffn):
    return (Linear("q", h, h), Linear("k", kv, h), Linear("v", kv, h), Linear("o", h, h),
            Linear("gate", ffn, h), Linear("up", ffn, h), Linear("down", h, ffn))


WORKLOADS = {
    "single": Workload("single", (Linear("w", 4096, 4096),), 16, 16, 32.0, "gauss", 0.02),
    "llama8b": Workload("llama8b", _llama_layer(4096, 1024, 14336), 2048, 16, 32.0, "gauss", 0.02),
    "llama65b": Workload("llama65b", _llama_layer(8192, 8192, 22016), 4096, 64, 16.0,
                         "gauss_outlier", 0.015),
    "llama70b": Workload("llama70b", _llama_layer(8192, 1024, 28672), 4096, 64, 16.0,
                         "student_t4", 0.015),
}
# Bandwidth workload: 136 matrices of 4096 x 14336 (7.986e9 weights) served from a pool of 8
# distinct seeded matrices, plus the skinny forward on one 8192 x 28672 weight.
STREAM_SHAPE = (4096, 14336)
STREAM_COUNT = 136
STREAM_POOL = 8
SKINNY = Workload("stream", (Linear("skinny", 8192, 28672),), 16, 16, 32.0, "gauss", 0.02)
SKINNY_MS = (1, 4, 16)


def rng_for(workload: str, linear: int, tensor: str, extra: int = 0) -> np.random.Generator:
    """A generator keyed by (workload, linear index, tensor, extra) under SeedSequence(0)."""
    ss = np.random.SeedSequence(entropy=0, spawn_key=(WORKLOAD_IDS[workload], linear,
                                                      TENSOR_IDS[tensor], extra))
    return np.random.Generator(np.random.PCG64(ss))


def weight(workload: str, linear: int, n: int, k: int, kind: str = "gauss",
           sigma: float = 0.02, extra: int = 0) -> np.ndarray:
    """A float32 N x K weight with the workload's value distribution."""
    g = rng_for(workload, linear, "w", extra)
    if kind == "gauss":
        w = g.standard_normal((n, k), dtype=np.float32) * np.float32(sigma)
    elif kind == "gauss_outlier":
        w = g.standard_normal((n, k), dtype=np.float32) * np.float32(sigma)
        cnt = int(round(0.001 * n * k))
        pos = g.choice(n * k, size=cnt, replace=False)
        w.reshape(-1)[pos] *= np.float32(20.0)
    elif kind == "student_t4":
        t = g.standard_t(4, size=(n, k))
        w = (t * (sigma / math.sqrt(2.0))).astype(np.float32)
    else:
        raise ValueError(kind)
    return w


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 with torch's cast and return the raw uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def gaussian_bf16(workload: str, linear: int, tensor: str, shape, sigma: float,
                  extra: int = 0) -> np.ndarray:
    g = rng_for(workload, linear, tensor, extra)
    a = g.standard_normal(shape, dtype=np.float32) * np.float32(sigma)
    return to_bf16_bits(a)


def linear_inputs(wl: Workload, li: int, lin: Linear, m: int | None = None):
    """(W fp32 [N,K], X bf16 [M,K], A bf16 [r,K], B bf16 [N,r], dY bf16 [M,N]) for one linear."""
    m = wl.m if m is None else m
    w = weight(wl.name, li, lin.n, lin.k, wl.weight_kind, wl.sigma)
    x = gaussian_bf16(wl.name, li, "x", (m, lin.k), 1.0)
    a = gaussian_bf16(wl.name, li, "a", (wl.r, lin.k), 0.01)
    b = gaussian_bf16(wl.name, li, "b", (lin.n, wl.r), 0.01)
    dy = gaussian_bf16(wl.name, li, "dy", (m, lin.n), 1.0)
    return w, x, a, b, dy


LLAMA8B_LAYERS = 32


def adapter_shapes(wl: Workload, layers: int = 1) -> list:
    """Shapes of the trainable tensors, layer by layer: A (r x K) then B (N x r) of every linear."""
    out = []
    for _ in range(layers):
        for lin in wl.linears:
            out += [(wl.r, lin.k), (lin.n, wl.r)]
    return out


def adapter_masters(workload: str, shapes, sigma: float = 0.01) -> list:
    """fp32 master weights of the adapters, one seeded stream per tensor."""
    return [rng_for(workload, i, "master").standard_normal(s, dtype=np.float32) * np.float32(sigma)
            for i, s in enumerate(shapes)]


def adapter_grads(workload: str, shapes, step: int, sigma: float = 1e-3) -> list:
    """fp32 adapter gradients of one step, one seeded stream per tensor and step."""
    return [rng_for(workload, i, "grad", step).standard_normal(s, dtype=np.float32) * np.float32(sigma)
            for i, s in enumerate(shapes)]


def stream_weight(i: int) -> np.ndarray:
    """Matrix i of the bandwidth stream (drawn from a pool of STREAM_POOL distinct matrices)."""
    return weight("stream", 100 + (i % STREAM_POOL), *STREAM_SHAPE, "gauss", 0.02)
