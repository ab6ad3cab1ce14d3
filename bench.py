"""Benchmark of the NF4 QLoRA linear layer on one MI355X.

A step is one forward + backward (dX, dA, dB) through all seven NF4 linears of a Llama-3.1-8B
layer (q/o 4096x4096, k/v 1024x4096, gate/up 14336x4096, down 4096x14336) at 2048 tokens, LoRA
rank 16, alpha 32: the training hot path, in which each weight is dequantised twice per step
inside the fused GEMMs. `value` is the algorithmic fwd+bwd TFLOP/s of the whole step, with inputs
already resident in HBM.

The same run also measures, each in its own timed loop:
  * the fused forward GEMM kernel alone (one launch per call through the forward-recompute entry),
    for the roofline against the bf16 dense MFMA peak;
  * quantise, double quantise and dequantise over 136 matrices of 4096 x 14336 (7.99e9 weights)
    drawn from a pool of 8 distinct matrices, the skinny forward of an 8192 x 28672 weight at
    1, 4 and 16 tokens with 4 rotating weight copies, and the adapter merge into that weight, in
    HBM GB/s against 8 TB/s;
  * the CPU oracle on a bounded sample of the same workload (cpu_baseline);
  * the other layer sets in `configs`: the single 4096x4096 linear at 16 tokens, and the 65B- and
    70B-shaped sets at 4096 tokens, rank 64 (step and fused forward GEMM).

Prints one JSON line. Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
METRIC = "QLoRA NF4 linear fwd+bwd TFLOP/s (% bf16 MFMA peak); NF4 dequant HBM GB/s"


def flops_fwd_bwd(n: int, k: int, m: int, r: int) -> int:
    """Forward 2MNK + 2Mr(K+N); backward dX 2MNK + 2Mr(N+K), dA 2rMK, dB 2NMr."""
    return (2 * m * n * k + 2 * m * r * (k + n)) + (2 * m * n * k + 2 * m * r * (n + k)
                                                    + 2 * r * m * k + 2 * n * m * r)


def nf4_bytes(numel: int) -> int:
    nb = numel // 64
    return numel // 2 + nb + 4 * ((nb + 255) // 256)


ROOFLINE_KERNEL = "qlora_gemm_kernel<false, 256, false>"


# Linears that share their input run their forward as one grouped launch (qlora_linear_fwd_group):
# a layer's query, key and value projections, and its gate and up projections.
GROUPS = (("q", "k", "v"), ("gate", "up"))


def fwd_tile_rows(m: int, n: int) -> int:
    """Token rows per tile of the fused forward GEMM, as its launcher picks them: 256 when there
    are more than 128 tokens and at least 192 such tiles of 128 output columns, else 128 above 64
    tokens, else 64."""
    tiles256 = -(-n // 128) * -(-m // 256)
    if m > 128 and tiles256 >= 192:
        return 256
    return 128 if m > 64 else 64


def copy_calibration():
    """A plain elementwise kernel of known traffic (fp32 negation, 1 GiB read, 1 GiB written),
    run under the same HBM counters as the GEMM to scale FETCH_SIZE and WRITE_SIZE to bytes."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"kernel": "torch neg fp32", "read_bytes": 4 * n,
                                           "write_bytes": 4 * n, "launches": 3}}), flush=True)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# what the dominant kernel (the fused GEMM) is built from: its sources and the compile flags
ROOFLINE_KERNEL_SOURCES = ("gemm.hip", "common.h")


def kernel_source_hash() -> str:
    from bit_nf4_quantised_amd import build as nf4_build
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_nf4_quantised_amd", "csrc")
    for name in ROOFLINE_KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    h.update(" ".join(nf4_build.COMMON).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel_key: str):
    """HBM bytes per launch of a kernel, from the committed rocprofv3 counter summary, if it was
    taken from the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    ent = t.get("kernels", {}).get(kernel_key)
    return None if ent is None else ent.get("bytes_per_launch")


def timed(fn, iters, torch):
    """Average milliseconds per call of fn() with HIP events on the current stream."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for i in range(iters):
        fn(i)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


def library_dense_gemm(torch, dev, m, lins, iters):
    """TFLOP/s of torch.matmul (hipBLASLt) on plain bf16 operands of the same shapes, with no
    quantisation: what a dense bf16 GEMM of these shapes sustains on this GPU. Context for the
    roofline only; nothing on the measured path uses it."""
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    xs = [torch.randn(m, l.k, device=dev, dtype=torch.bfloat16, generator=g) for l in lins]
    ws = [torch.randn(l.n, l.k, device=dev, dtype=torch.bfloat16, generator=g) * 0.02 for l in lins]

    def run(_i=0):
        for x, w in zip(xs, ws):
            torch.matmul(x, w.t())

    run()
    ms = timed(run, iters, torch)
    return sum(2 * m * l.n * l.k for l in lins) / (ms * 1e-3) / 1e12


def prepare(wk, q, dev, torch):
    """Every linear's inputs resident in HBM: the NF4 weight (quantised on the GPU), x, A, B, dY and
    the outputs. The seeded host generators run in a thread pool (numpy fills arrays without the
    interpreter lock), one linear per thread."""
    from concurrent.futures import ThreadPoolExecutor
    M, r = wk.m, wk.r
    lin_state, ws_bytes, flops = [], 0, 0
    t16 = lambda arr: torch.from_numpy(arr.view(np.int16)).to(dev)  # noqa: E731
    with ThreadPoolExecutor(max_workers=min(8, len(wk.linears))) as ex:
        futs = [ex.submit(wl.linear_inputs, wk, li, lin) for li, lin in enumerate(wk.linears)]
        for lin, fut in zip(wk.linears, futs):
            w, x, a, b, dy = fut.result()
            wt = torch.from_numpy(w).to(dev)
            del w
            qw = q.quantize_weight(wt)
            del wt
            lin_state.append(dict(lin=lin, qw=qw, x=t16(x), a=t16(a), b=t16(b), dy=t16(dy),
                                  y=torch.empty(M, lin.n, dtype=torch.int16, device=dev),
                                  u=torch.empty(M, r, dtype=torch.float32, device=dev),
                                  dx=torch.empty(M, lin.k, dtype=torch.int16, device=dev),
                                  dA=torch.empty(r, lin.k, dtype=torch.float32, device=dev),
                                  dB=torch.empty(lin.n, r, dtype=torch.float32, device=dev)))
            ws_bytes = max(ws_bytes, q.qlora_workspace_bytes(M, lin.n, lin.k, r))
            flops += flops_fwd_bwd(lin.n, lin.k, M, r)
    # units of the step: the groups (members share the first member's x, as the projections of one
    # layer input do), then every other linear on its own, in the order of their first linear
    by_name = {st["lin"].name: st for st in lin_state}
    grouped = set()
    units = []
    for st in lin_state:
        name = st["lin"].name
        if name in grouped:
            continue
        unit = [st]
        for grp in GROUPS:
            if name == grp[0] and all(n in by_name for n in grp) and \
                    len({by_name[n]["lin"].k for n in grp}) == 1:
                unit = [by_name[n] for n in grp]
                for other in unit[1:]:
                    other["x"] = st["x"]
                grouped.update(grp)
                ws_bytes = max(ws_bytes, q.qlora_workspace_bytes_group(M, [u["lin"].n for u in unit], st["lin"].k, r))
        units.append(unit)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    return units, ws, flops


def fwd_unit(q, unit, s, ws):
    """The forward of one unit: a grouped launch, or one linear."""
    if len(unit) > 1:
        q.qlora_linear_fwd_group([st["qw"] for st in unit], unit[0]["x"], [st["a"] for st in unit],
                                 [st["b"] for st in unit], s, [st["y"] for st in unit], [st["u"] for st in unit],
                                 ws=ws)
    else:
        st = unit[0]
        q.qlora_linear_fwd(st["qw"], st["x"], st["a"], st["b"], s, st["y"], st["u"], ws=ws)


def bwd_unit(q, unit, s, ws):
    """The backward of one unit: a grouped backward (one dX launch for the group), or one linear."""
    if len(unit) > 1:
        q.qlora_linear_bwd_group([st["qw"] for st in unit], unit[0]["x"], [st["dy"] for st in unit],
                                 [st["a"] for st in unit], [st["b"] for st in unit], s, [st["u"] for st in unit],
                                 [st["dx"] for st in unit], [st["dA"] for st in unit], [st["dB"] for st in unit],
                                 ws=ws)
    else:
        st = unit[0]
        q.qlora_linear_bwd(st["qw"], st["x"], st["dy"], st["a"], st["b"], s, st["u"], st["dx"],
                           st["dA"], st["dB"], ws=ws)


def step_fn(q, units, ws, s):
    def step(_i=0):
        for unit in units:
            fwd_unit(q, unit, s, ws)
            bwd_unit(q, unit, s, ws)
    return step


def unit_name(unit):
    return "+".join(st["lin"].name for st in unit)


def unit_tile_rows(M, unit):
    """Token rows per tile of a unit's forward GEMM: a group of linears takes 256-row tiles when
    their tiles together number at least 192 (above 128 tokens), as the grouped launcher decides."""
    if len(unit) > 1:
        tiles = sum(-(-st["lin"].n // 128) for st in unit) * -(-M // 256)
        return 256 if M > 128 and tiles >= 192 else 0
    return fwd_tile_rows(M, unit[0]["lin"].n)


def fwd_gemm_fn(q, units, M, s, weights=None):
    """The forward GEMMs of the units whose forward runs the 256-row tile instantiation, as the step
    launches them (a group as one launch), through the forward-recompute entries; returns (fn,
    units, flops per call). `weights` maps linear names to other quantised weights of the same
    shapes (default: each linear's own)."""
    r = units[0][0]["a"].shape[0]
    big = [u for u in units if unit_tile_rows(M, u) == 256]
    w = (lambda st: weights[st["lin"].name]) if weights else (lambda st: st["qw"])  # noqa: E731

    def recompute(_i=0):
        for unit in big:
            if len(unit) > 1:
                q.qlora_linear_fwd_recompute_group([w(st) for st in unit], unit[0]["x"], [st["a"] for st in unit],
                                                   [st["b"] for st in unit], s, [st["u"] for st in unit],
                                                   [st["y"] for st in unit])
            else:
                st = unit[0]
                q.qlora_linear_fwd_recompute(w(st), st["x"], st["a"], st["b"], s, st["u"], st["y"])
    flops = sum(2 * M * st["lin"].n * (st["lin"].k + r) for u in big for st in u)
    return recompute, big, flops


def other_configs(torch, q, dev, skip):
    """The other layer sets at their own shapes, each timed in a short loop after one untimed step:
    the 16-token single linear (latency-bound: microseconds per step), and the 65B- and 70B-shaped
    sets at 4096 tokens and rank 64 (step TFLOP/s and the fused forward GEMM alone)."""
    out = {}
    for name in ("single", "llama65b", "llama70b"):
        if name == skip:
            continue
        wk = wl.WORKLOADS[name]
        log(f"[bench] config {name}: preparing {len(wk.linears)} linears, M={wk.m}, r={wk.r}")
        units, ws, flops = prepare(wk, q, dev, torch)
        step = step_fn(q, units, ws, wk.scale)
        step()
        iters = 50 if name == "single" else 3
        ms = timed(step, iters, torch)
        tf = flops / (ms * 1e-3) / 1e12
        ent = {"linears": {l.name: [l.n, l.k] for l in wk.linears}, "tokens": wk.m, "rank": wk.r,
               "alpha": wk.alpha, "weights": wk.weight_kind, "flops_per_step": flops,
               "ms_per_step": round(ms, 4), "TFLOPs": round(tf, 2),
               "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "steps": iters}
        if name == "single":
            nf4 = sum(nf4_bytes(l.n * l.k) for l in wk.linears)
            ent.update({"us_per_step": round(ms * 1e3, 2),
                        "nf4_GBps": round(2 * nf4 / (ms * 1e-3) / 1e9, 1),
                        "nf4_bytes_per_step": 2 * nf4,
                        "what": "forward (few-token kernel) + backward (dX GEMM, dA, dB) of one "
                                "4096x4096 linear at 16 tokens; the weight is read twice per step"})
            log(f"[bench] config single: {ms*1e3:.1f} us per fwd+bwd")
            # the same step captured in a HIP graph (every call is a plain sequence of kernel
            # launches): ten steps per graph, replayed, so that the host's launch work per kernel
            # leaves the measured time; the eager figure above is the primary one
            reps = 10
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(reps):
                    step(i)
            graph.replay()
            ms_g = timed(lambda _i: graph.replay(), 5, torch) / reps
            ent["us_per_step_hip_graph"] = round(ms_g * 1e3, 2)
            log(f"[bench] config single, replayed from a HIP graph: {ms_g*1e3:.1f} us per fwd+bwd")
            del graph
        else:
            fwd, big, gflops = fwd_gemm_fn(q, units, wk.m, wk.scale)
            fwd()
            ms_f = timed(fwd, iters, torch)
            ach = gflops / (ms_f * 1e-3) / 1e12
            ent["fused_fwd_gemm"] = {"kernel": ROOFLINE_KERNEL, "achieved_TFLOPs": round(ach, 2),
                                     "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                                     "avg_launch_us": round(ms_f * 1e3 / len(big), 2),
                                     "launches": [unit_name(u) for u in big]}
            log(f"[bench] config {name}: step {ms:.2f} ms, {tf:.1f} TFLOP/s; fused fwd GEMM {ach:.1f} TFLOP/s")
        out[name] = ent
        del units, ws
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b", choices=["llama8b", "llama65b", "llama70b"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-paths", action="store_true", help="skip the bandwidth-path loops")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other layer sets (single linear, 65B- and 70B-shaped)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the known-size copy kernel used to scale HBM counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1 (the data-"
                                   "parallel sharding across GPUs is described, not built)"}))
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    import bit_nf4_quantised_amd as q

    dev = torch.device("cuda:0")
    wk = wl.WORKLOADS[args.workload]
    M, r, s = wk.m, wk.r, wk.scale

    # ---------------------------------------------------------------- step inputs, resident in HBM
    log(f"[bench] preparing {args.workload}: {len(wk.linears)} linears, M={M}, r={r}")
    units, ws, flops = prepare(wk, q, dev, torch)
    lin_state = [st for u in units for st in u]
    step = step_fn(q, units, ws, s)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms_per_step = timed(step, args.steps, torch)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    log(f"[bench] step {ms_per_step:.3f} ms, {tflops:.1f} TFLOP/s")

    # ------------------------------------------------ dominant kernel: fused forward GEMM, alone
    # Timed over the forward launches of the 256-row tile instantiation qlora_gemm_kernel<false,
    # 256, false>, as the step issues them (a group as one launch), so that the average launch
    # matches that kernel's entry in a rocprofv3 kernel-trace summary of this same command.
    recompute, big, gemm_flops = fwd_gemm_fn(q, units, M, s)
    recompute()
    ms_recompute = timed(recompute, args.steps, torch)
    launches = len(big)
    avg_launch_ms = ms_recompute / launches
    gemm_achieved = gemm_flops / (ms_recompute * 1e-3) / 1e12
    traffic = load_traffic(ROOFLINE_KERNEL)
    roofline = {"kernel": ROOFLINE_KERNEL + " (forward: fused NF4 dequant + bf16 MFMA + adapter)",
                "bound": "mfma", "achieved": round(gemm_achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(gemm_achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "avg_launch_us": round(avg_launch_ms * 1e3, 2),
                "flops_per_launch": gemm_flops // launches,
                "launches": [unit_name(u) for u in big]}
    log(f"[bench] fused fwd GEMM {gemm_achieved:.1f} TFLOP/s, {avg_launch_ms*1e3:.1f} us/launch")
    # the same forward GEMMs on weights that keep fp32 scales (no double quantisation)
    f32s = {}
    for unit in big:
        for st in unit:
            li = wk.linears.index(st["lin"])
            wt = torch.from_numpy(wl.linear_inputs(wk, li, st["lin"], m=1)[0]).to(dev)
            f32s[st["lin"].name] = q.quantize_weight(wt, double_quant=False)
            del wt
    recompute_f32s, _, _ = fwd_gemm_fn(q, units, M, s, weights=f32s)
    recompute_f32s()
    ms_f32s = timed(recompute_f32s, args.steps, torch)
    fwd_f32s = {"TFLOPs": round(gemm_flops / (ms_f32s * 1e-3) / 1e12, 2),
                "vs_double_quantised": round(ms_recompute / ms_f32s, 4),
                "what": "the roofline kernel's forward GEMMs with fp32 absmax scales instead of "
                        "double-quantised ones (4.5 instead of 4.127 bits per weight)"}
    log(f"[bench] fused fwd GEMM, fp32 scales: {fwd_f32s['TFLOPs']:.1f} TFLOP/s")
    del f32s
    # a group as one GEMM of its stacked weights
    shapes = [SimpleNamespace(n=sum(st["lin"].n for st in u), k=u[0]["lin"].k) for u in big]
    dense = library_dense_gemm(torch, dev, M, shapes, args.steps)
    log(f"[bench] library dense bf16 GEMM, same shapes: {dense:.1f} TFLOP/s")
    context = {"library_dense_bf16_gemm_TFLOPs": round(dense, 2),
               "fused_vs_library_dense": round(gemm_achieved / dense, 4),
               "what": "torch.matmul (hipBLASLt) on plain bf16 operands of the roofline kernel's "
                       "shapes, no quantisation, timed the same way: the dense GEMM rate this GPU "
                       "sustains at these shapes"}

    paths = {}
    dequant_gbps = None
    if not args.no_paths:
        paths, dequant_gbps = bandwidth_paths(torch, q, dev, args)
    group_names = [unit_name(u) for u in units if len(u) > 1]
    del lin_state, units, ws
    torch.cuda.empty_cache()
    configs = {} if args.no_configs else other_configs(torch, q, dev, args.workload)

    cpu = None if args.no_cpu_baseline else cpu_baseline(wk)

    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; weights N(0,0.02^2), x and dY N(0,1) with one x per layer input (q/k/v share one, gate/up another), A and B N(0,0.01^2))",
        "config": {"workload": f"{args.workload} layer set, all 7 linears NF4 + double quant, "
                               f"fwd + bwd (dX, dA, dB)",
                   "tokens": M, "rank": r, "alpha": wk.alpha,
                   "linears": {l.name: [l.n, l.k] for l in wk.linears},
                   "grouped": group_names,
                   "flops_per_step": flops},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "dequant_GBps": dequant_gbps,
        "roofline": roofline,
        "context": context,
        "cpu_baseline": cpu,
        "paths": paths,
        "fwd_gemm_fp32_scales": fwd_f32s,
        "configs": configs,
    }
    print(json.dumps(out), flush=True)


def bandwidth_paths(torch, q, dev, args):
    """Quantise / double-quantise / dequantise over the 136-matrix stream, and the skinny forward."""
    res = {}
    n_rows, n_cols = wl.STREAM_SHAPE
    numel = n_rows * n_cols
    nb = numel // 64
    log(f"[bench] stream pool: {wl.STREAM_POOL} x {n_rows}x{n_cols} fp32")
    pool = [torch.from_numpy(wl.stream_weight(i)).to(dev) for i in range(wl.STREAM_POOL)]
    qws = [q.empty_weight(n_rows, n_cols, dev) for _ in range(wl.STREAM_POOL)]
    absmax = [torch.empty(nb, dtype=torch.float32, device=dev) for _ in range(wl.STREAM_POOL)]
    outs = [torch.empty(numel, dtype=torch.int16, device=dev) for _ in range(2)]
    count = wl.STREAM_COUNT

    def quant(i):
        j = i % wl.STREAM_POOL
        q.nf4_quantize(pool[j], qws[j].packed, absmax[j])

    def dq(i):
        j = i % wl.STREAM_POOL
        q.nf4_double_quant(absmax[j], qws[j].scale_q, qws[j].scale_c2)

    def deq(i):
        q.nf4_dequant(qws[i % wl.STREAM_POOL], outs[i % 2])

    for fn in (quant, dq, deq):
        fn(0)
    torch.cuda.synchronize()
    total = count * numel
    ng = (nb + 255) // 256
    # double quantisation of all 136 matrices' scales through one nf4_double_quant_many call
    # (64 matrices per launch), as a model's weights are processed at load time
    # every matrix with its own scales and outputs (copies of its pool matrix's scales), as a
    # model's weights have: 0.5 GB of scales in, 0.13 GB of codes and constants out
    dq_in = [absmax[i % wl.STREAM_POOL].clone() for i in range(count)]
    dq_q = [torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(count)]
    dq_c2 = [torch.empty(ng, dtype=torch.float32, device=dev) for _ in range(count)]
    dq_many = q.DoubleQuantMany(dq_in, dq_q, dq_c2)
    dq_many()
    for name, fn, calls, reps, per_weight_bytes in (
            ("quantize", quant, count, 1, 4 + 0.5 + 4 / 64),
            ("double_quant", lambda _i: dq_many(), 1, 10, (4 * nb + nb + 4 * ng) / numel),
            ("dequant", deq, count, 1, nf4_bytes(numel) / numel + 2)):
        ms = timed(fn, calls * reps, torch) * calls   # ms for the whole stream
        gbps = total * per_weight_bytes / (ms * 1e-3) / 1e9
        res[name] = {"weights": total, "ms_total": round(ms, 3),
                     "GBps": round(gbps, 1), "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4),
                     "bytes_per_weight": round(per_weight_bytes, 4)}
        log(f"[bench] {name}: {gbps:.0f} GB/s")
    # one nf4_double_quant call per matrix, for comparison (launch-bound)
    ms = timed(dq, count, torch)
    res["double_quant"]["one_call_per_matrix_GBps"] = round(
        total * (4 * nb + nb + 4 * ng) / numel / (ms * count * 1e-3) / 1e9, 1)
    del dq_many, dq_in, dq_q, dq_c2
    dequant_gbps = res["dequant"]["GBps"]

    # codebook and blocksize variants over the same pool: quantise, and dequantise with fp32 scales
    # (no double quantisation), 16 launches each (two passes over the pool)
    variants = {}
    nvar = 16
    for book, bs in (("nf4", 64), ("fp4", 64), ("int4", 64), ("nf4", 16), ("nf4", 4096)):
        am = [torch.empty(numel // bs, dtype=torch.float32, device=dev) for _ in range(wl.STREAM_POOL)]

        def vq(i, book=book, bs=bs, am=am):
            j = i % wl.STREAM_POOL
            q.q4_quantize(pool[j], book, bs, qws[j].packed, am[j])

        def vd(i, book=book, bs=bs, am=am):
            j = i % wl.STREAM_POOL
            q.q4_dequant(qws[j].packed, numel, book, bs, outs[i % 2], absmax=am[j])

        for i in range(wl.STREAM_POOL):
            vq(i)
        torch.cuda.synchronize()
        ent = {}
        for name, fn, per_weight in (("quantize", vq, 4 + 0.5 + 4 / bs), ("dequant_fp32_scales", vd, 0.5 + 4 / bs + 2)):
            ms = timed(fn, nvar, torch)
            gbps = numel * per_weight / (ms * 1e-3) / 1e9
            ent[name] = {"GBps": round(gbps, 1), "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4),
                         "bytes_per_weight": round(per_weight, 4), "us_per_matrix": round(ms * 1e3, 2)}
        variants[f"{book}_bs{bs}"] = ent
        log(f"[bench] variant {book} bs {bs}: quantise {ent['quantize']['GBps']:.0f} GB/s, "
            f"dequantise {ent['dequant_fp32_scales']['GBps']:.0f} GB/s")
        del am
    res["variants_4096x14336"] = variants
    del pool, qws, absmax, outs
    torch.cuda.empty_cache()

    # skinny forward: 8192 x 28672, rank 16, 4 rotating copies of the quantised weight (> MALL)
    sk = wl.SKINNY
    lin = sk.linears[0]
    log("[bench] skinny weight 8192x28672")
    w = wl.weight("stream", 0, lin.n, lin.k, "gauss", 0.02)
    base = q.quantize_weight(torch.from_numpy(w).to(dev))
    base_f32 = q.quantize_weight(torch.from_numpy(w).to(dev), double_quant=False)
    del w
    copies = [base] + [q.NF4Weight(base.packed.clone(), base.scale_q.clone(), base.scale_c2.clone(),
                                   base.N, base.K) for _ in range(3)]
    skinny = {}
    for m in wl.SKINNY_MS:
        _, x, a, b, _ = wl.linear_inputs(sk, 0, lin, m=m)
        t16 = lambda arr: torch.from_numpy(arr.view(np.int16)).to(dev)
        X, A, B = t16(x), t16(a), t16(b)
        y = torch.empty(m, lin.n, dtype=torch.int16, device=dev)
        u = torch.empty(m, sk.r, dtype=torch.float32, device=dev)
        wsk = q.workspace(m, lin.n, lin.k, sk.r, dev)

        def call(i):
            q.qlora_linear_fwd(copies[i % len(copies)], X, A, B, sk.scale, y, u, ws=wsk)

        call(0)
        ms = timed(call, 200, torch)
        nbytes = (nf4_bytes(lin.n * lin.k) + 2 * m * lin.k + 2 * sk.r * lin.k + 2 * lin.n * sk.r
                  + 2 * m * lin.n + 4 * m * sk.r)
        gbps = nbytes / (ms * 1e-3) / 1e9
        skinny[f"M={m}"] = {"us": round(ms * 1e3, 2), "GBps": round(gbps, 1),
                            "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4), "bytes": nbytes}
        log(f"[bench] skinny M={m}: {ms*1e3:.1f} us, {gbps:.0f} GB/s")
        if m in (1, 16):
            # the same forward with fp32 block scales (no double quantisation), 4 rotating copies
            fcopies = [base_f32] + [q.NF4Weight(base_f32.packed.clone(), None, None, base_f32.N, base_f32.K,
                                                absmax=base_f32.absmax.clone()) for _ in range(3)]

            def fcall(i):
                q.qlora_linear_fwd(fcopies[i % len(fcopies)], X, A, B, sk.scale, y, u, ws=wsk)

            fcall(0)
            fms = timed(fcall, 200, torch)
            fbytes = nbytes - nf4_bytes(lin.n * lin.k) + lin.n * lin.k // 2 + 4 * (lin.n * lin.k // 64)
            skinny[f"M={m} fp32 scales"] = {"us": round(fms * 1e3, 2), "GBps": round(fbytes / (fms * 1e-3) / 1e9, 1),
                                            "frac_hbm": round(fbytes / (fms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                                            "bytes": fbytes}
            log(f"[bench] skinny M={m}, fp32 scales: {fms*1e3:.1f} us")
            del fcopies
    res["skinny_fwd_8192x28672"] = skinny
    del base_f32

    # adapter merge into the dequantised base, same weight (4 rotating copies), rank 16
    _, _, a, b, _ = wl.linear_inputs(sk, 0, lin, m=1)
    A = torch.from_numpy(a.view(np.int16)).to(dev)
    B = torch.from_numpy(b.view(np.int16)).to(dev)
    merged = torch.empty(lin.n * lin.k, dtype=torch.int16, device=dev)

    def merge_call(i):
        q.qlora_merge(copies[i % len(copies)], A, B, sk.scale, merged)

    merge_call(0)
    ms = timed(merge_call, 50, torch)
    nbytes = nf4_bytes(lin.n * lin.k) + 2 * lin.n * lin.k + 2 * sk.r * lin.k + 2 * lin.n * sk.r
    gbps = nbytes / (ms * 1e-3) / 1e9
    res["merge_8192x28672_r16"] = {"us": round(ms * 1e3, 2), "GBps": round(gbps, 1),
                                   "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4), "bytes": nbytes}
    log(f"[bench] merge: {ms*1e3:.1f} us, {gbps:.0f} GB/s")
    del copies, base, merged
    torch.cuda.empty_cache()
    res["adapter_update_llama8b"] = adapter_update_path(torch, q, dev)
    return res, dequant_gbps


def adapter_update_path(torch, q, dev, iters=50):
    """The adapter update of a training step over every adapter of a 32-layer Llama-3.1-8B at
    rank 16 (448 tensors, 41.9 M values), through one plan: the global gradient norm, then clipped
    AdamW with fp32 state and bf16 copies of the new weights. Per value 34 bytes: the norm pass
    reads the gradient (4); the step reads p, g, m, v (16) and writes p, m, v (12) and the bf16
    copy (2)."""
    shapes = wl.adapter_shapes(wl.WORKLOADS["llama8b"], wl.LLAMA8B_LAYERS)
    log(f"[bench] adapter update: {len(shapes)} tensors")
    p = [torch.from_numpy(x).to(dev) for x in wl.adapter_masters("llama8b", shapes)]
    g = [torch.from_numpy(x).to(dev) for x in wl.adapter_grads("llama8b", shapes, 1)]
    m = [torch.zeros_like(x) for x in p]
    v = [torch.zeros_like(x) for x in p]
    pb = [torch.empty(x.numel(), dtype=torch.int16, device=dev) for x in p]
    norm = torch.empty(1, dtype=torch.float64, device=dev)
    plan = q.AdamWPlan(p, g, m, v, pb, q.AdamWConfig())
    plan.step(1, norm)
    ms = timed(lambda i: plan.step(i + 2, norm), iters, torch)
    values = plan.values
    nbytes = 34 * values
    gbps = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] adapter update: {ms*1e3:.1f} us, {gbps:.0f} GB/s, grad norm {float(norm.cpu()):.3f}")
    plan.close()
    return {"tensors": len(shapes), "values": values, "us": round(ms * 1e3, 2), "GBps": round(gbps, 1),
            "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4), "bytes": nbytes, "launches": 3}


def cpu_baseline(wk, min_seconds: float = 10.0):
    """The oracle, as it stands, on a bounded sample of the workload: quantise + double-quantise +
    dequantise, forward and backward of every linear of the layer set at full token count, in
    whole passes over the layer set until at least `min_seconds` of oracle time have run."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    sample = list(range(len(wk.linears)))
    inputs = {}
    flops = 0
    secs = 0.0
    passes = 0
    while passes == 0 or secs < min_seconds:
        for li in sample:
            lin = wk.linears[li]
            if li not in inputs:                      # input generation is not timed
                inputs[li] = wl.linear_inputs(wk, li, lin)
            w, x, a, b, dy = inputs[li]
            t_start = time.perf_counter()
            packed, c1 = oracle.quantize(w)
            codes, c2 = oracle.double_quant(c1)
            wt = oracle.dequant(packed, codes, c2, w.size).reshape(lin.n, lin.k)
            oracle.linear_fwd(x, wt, a, b, wk.scale)
            oracle.linear_bwd(x, dy, wt, a, b, wk.scale)
            secs += time.perf_counter() - t_start
            flops += flops_fwd_bwd(lin.n, lin.k, wk.m, wk.r)
        passes += 1
        log(f"[bench] cpu oracle pass {passes}: cumulative {secs:.1f} s")
    return _cpu_result(flops, secs, threads, sample, wk, passes)


def _cpu_result(flops, secs, threads, sample, wk, passes):
    names = "+".join(wk.linears[i].name for i in sample)
    return {"value": round(flops / secs / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": round(secs, 2),
            "sample": f"{passes} pass(es) over the {names} linears of {wk.name} (M={wk.m}, "
                      f"r={wk.r}): NF4 quantise, double quantise, dequantise, fp64 forward and "
                      f"backward; fwd+bwd flops / oracle wall time"}


if __name__ == "__main__":
    main()
