"""Turn the rocprofv3 CSV output of the profiling commands below (each writes into the directory
its -d option names) into the text summaries under profiles/, and record the fused GEMM's HBM bytes
per launch in profiles/traffic.json with a hash of that kernel's sources, which bench.py reads for
its roofline's traffic field.

    python3 profile_summary.py "<workload description>"
"""
import collections
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

OUT = os.path.join(ROOT, "gpurun_out")
PROF = os.path.join(ROOT, "profiles")

KTRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/ktrace -o run -- "
              "python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-paths")
PMC_CMD = ("timeout -s KILL 240 rocprofv3 --pmc {c} --output-format csv -d gpurun_out/pmc_{d} -o run -- "
           "python3 bench.py --steps 2 --warmup 0 --no-cpu-baseline --no-paths")
COPY_CMD = ("timeout -s KILL 120 rocprofv3 --pmc {c} --output-format csv -d gpurun_out/pmc_copy_{d} "
            "-o run -- python3 bench.py --copy-calibration")


def short(name):
    return name.split("(")[0].replace("void ", "").replace("nf4::", "")


def ktrace(tag, bench_json):
    stats = list(csv.DictReader(open(f"{OUT}/ktrace/run_kernel_stats.csv")))
    rows = list(csv.DictReader(open(f"{OUT}/ktrace/run_kernel_trace.csv")))
    per = collections.defaultdict(list)
    for r in rows:
        g = (short(r["Kernel_Name"]), int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]),
             int(r["Grid_Size_Y"]))
        per[g].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    b = json.load(open(bench_json))
    lines = [f"# Kernel trace: {tag}", "",
             "Command (from the repository root, on one MI355X):", "", "```", KTRACE_CMD, "```", "",
             "## rocprofv3 --stats (all kernels of the command)", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for s in stats:
        lines.append(f"| `{short(s['Name'])}` | {s['Calls']} | {float(s['AverageNs'])/1e3:.1f} | "
                     f"{float(s['MinNs'])/1e3:.1f} | {float(s['MaxNs'])/1e3:.1f} | {s['Percentage']} |")
    lines += ["", "## Per launch shape (grid in workgroups x, y)", "",
              "| kernel | grid | launches | median us | min us | total us |", "|---|---|---|---|---|---|"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        v2 = sorted(v)
        lines.append(f"| `{k[0]}` | {k[1]} x {k[2]} | {len(v)} | {v2[len(v2)//2]:.1f} | {v2[0]:.1f} | "
                     f"{sum(v):.1f} |")
    rl = b["roofline"]
    st = [s for s in stats if short(s["Name"]) == "qlora_gemm_kernel<false, 256, false>"][0]
    lines += ["", "## Agreement with the benchmark's live measurement", "",
              f"`bench.py` (default run, HIP events over its timed forward loop) reports "
              f"{rl['avg_launch_us']} us per launch of `{bench.ROOFLINE_KERNEL}` averaged over "
              f"the {', '.join(rl['linears'])} linears; the trace above averages "
              f"{float(st['AverageNs'])/1e3:.1f} us over the same linears' launches in the step and "
              f"the forward loop ({st['Calls']} launches).", ""]
    return "\n".join(lines)


PATHS_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/ktrace_paths -o run -- "
             "python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline")
PATH_KERNELS = {
    "nf4_quantize_kernel": "quantise: 136 matrices of 4096x14336 (per weight 4.5625 B), plus the "
                           "setup quantisations of other shapes",
    "nf4_double_quant_kernel": "double quantise: same stream (per weight 0.0784 B), plus setup",
    "nf4_dequant_kernel": "dequantise, same stream (per weight 2.5159 B)",
    "skinny4_fwd_kernel<false>": "skinny forward, 8192x28672 at M = 1 and 4 (four rows x four chunks per MFMA)",
    "skinny4_fwd_kernel<true>": "the same at M = 1 with fp32 block scales (no double quantisation)",
    "skinny_fwd_kernel": "skinny forward, 8192x28672 at M = 16",
    "skinny_epilogue_kernel": "its split-K epilogue",
    "qlora_merge_kernel<1>": "adapter merge, 8192x28672, rank 16",
    "grad_sqnorm_partial_kernel": "adapter update, norm partial sums (448 tensors, 41.9 M values)",
    "grad_sqnorm_final_kernel": "adapter update, norm total",
    "adamw_kernel": "adapter update, clipped AdamW",
    "q4_quantize_kernel<16>": "variant quantise, blocksize 16 (NF4), 4096x14336 pool",
    "q4_quantize_kernel<64>": "variant quantise, blocksize 64 (NF4, FP4, INT4), 4096x14336 pool",
    "q4_quantize_kernel<4096>": "variant quantise, blocksize 4096 (NF4), 4096x14336 pool",
    "q4_dequant_kernel<4, false>": "variant dequantise, fp32 scales, blocksize 16",
    "q4_dequant_kernel<1, false>": "variant dequantise, fp32 scales, blocksizes 64 and 4096",
}


def paths_trace(tag):
    stats = list(csv.DictReader(open(f"{OUT}/ktrace_paths/run_kernel_stats.csv")))
    lines = [f"# Kernel trace of the bandwidth paths: {tag}", "",
             "Command (from the repository root, on one MI355X); the same run also holds the step's "
             "kernels, listed in the fused-GEMM trace:", "", "```", PATHS_CMD, "```", "",
             "| kernel | what | calls | avg us | min us | max us |", "|---|---|---|---|---|---|"]
    for s in stats:
        k = short(s["Name"])
        if k in PATH_KERNELS:
            lines.append(f"| `{k}` | {PATH_KERNELS[k]} | {s['Calls']} | {float(s['AverageNs'])/1e3:.1f} | "
                         f"{float(s['MinNs'])/1e3:.1f} | {float(s['MaxNs'])/1e3:.1f} |")
    lines.append("")
    return "\n".join(lines)


def pmc(name):
    rows = list(csv.DictReader(open(f"{OUT}/{name}/run_counter_collection.csv")))
    d = collections.defaultdict(list)
    for r in rows:
        d[(short(r["Kernel_Name"]), int(r["Grid_Size"]) // int(r["Workgroup_Size"]))].append(
            float(r["Counter_Value"]))
    return d


def counters(tag, bench_json):
    fetch, write = pmc("pmc_fetch"), pmc("pmc_write")
    cf, cw = pmc("pmc_copy_fetch"), pmc("pmc_copy_write")
    copy_bytes = 4 << 28
    cfv = max(v for vals in cf.values() for v in vals)   # the negation kernel (the fill reads ~0)
    cwv = [v for vals in cw.values() for v in vals]
    f_scale = copy_bytes / (cfv * 1024)
    w_scale = copy_bytes / (max(cwv) * 1024)
    b = json.load(open(bench_json))
    lines = [f"# HBM-side traffic counters: {tag}", "",
             "Commands (from the repository root, on one MI355X), one counter per pass:", "", "```",
             PMC_CMD.format(c="FETCH_SIZE", d="fetch"), PMC_CMD.format(c="WRITE_SIZE", d="write"),
             COPY_CMD.format(c="FETCH_SIZE", d="fetch"), COPY_CMD.format(c="WRITE_SIZE", d="write"),
             "```", "",
             "Calibration: the copy kernel (fp32 negation, 1 GiB read and 1 GiB written) reads "
             f"{cfv:.0f} KiB FETCH_SIZE and {max(cwv):.0f} KiB WRITE_SIZE per launch, so bytes = "
             f"FETCH_SIZE x 1024 x {f_scale:.3f} and WRITE_SIZE x 1024 x {w_scale:.3f}.", "",
             "FETCH_SIZE and WRITE_SIZE count L2 traffic to and from the memory fabric; reads that hit "
             "the memory-side cache are included.", "",
             "| kernel | grid WGs | launches | fetch MB/launch | write MB/launch |", "|---|---|---|---|---|"]
    for k in sorted(fetch, key=lambda k: -sum(fetch[k])):
        fv, wv = fetch[k], write.get(k, [0])
        lines.append(f"| `{k[0]}` | {k[1]} | {len(fv)} | {sum(fv)/len(fv)*1024*f_scale/1e6:.1f} | "
                     f"{sum(wv)/len(wv)*1024*w_scale/1e6:.1f} |")
    # the benchmark's roofline kernel: average over its forward loop's linears, one launch each
    rl = b["roofline"]
    wk = bench.wl.WORKLOADS["llama8b"]
    big = [l for l in wk.linears if bench.fwd_tile_rows(wk.m, l.n) == 256]
    key = "qlora_gemm_kernel<false, 256, false>"
    # q, o and down share one grid size; their mean stands for each of them
    tot_f = tot_w = 0.0
    for l in big:
        g = ((l.n + 127) // 128) * ((wk.m + 255) // 256)
        fv = fetch[(key, g)]
        wv = write[(key, g)]
        tot_f += sum(fv) / len(fv)
        tot_w += sum(wv) / len(wv)
    n = len(big)
    fb = tot_f / n * 1024 * f_scale
    wb = tot_w / n * 1024 * w_scale
    alg = 0
    for l in big:
        alg += (2 * wk.m * l.k + bench.nf4_bytes(l.n * l.k) + 2 * l.n * wk.r + 4 * wk.m * wk.r
                + 2 * wk.m * l.n)
    alg /= n
    lines += ["", f"## {key} (the benchmark's roofline kernel)", "",
              f"Mean over one launch of each of {', '.join(l.name for l in big)}: fetch "
              f"{fb/1e6:.1f} MB + write {wb/1e6:.1f} MB = {(fb+wb)/1e6:.1f} MB per launch, against "
              f"{alg/1e6:.1f} MB of algorithmic bytes (X, packed W with its scales, B, u, y).", ""]
    traffic = {"source_hash": bench.kernel_source_hash(),
               "calibration": {"fetch_scale": f_scale, "write_scale": w_scale},
               "kernels": {key: {"bytes_per_launch": int(fb + wb), "fetch_bytes": int(fb),
                                 "write_bytes": int(wb), "algorithmic_bytes": int(alg),
                                 "linears": [l.name for l in big]}}}
    return "\n".join(lines), traffic


CLOCK_CMD = ("timeout -s KILL 240 rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES "
             "--output-format csv -d gpurun_out/pmc_clock -o run -- python3 bench.py --steps 2 --warmup 0 "
             "--no-cpu-baseline --no-paths")


def clock(tag):
    rows = list(csv.DictReader(open(f"{OUT}/pmc_clock/run_counter_collection.csv")))
    d = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in rows:
        name = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("nf4::", "")
        if name.startswith("Cijk") or name.startswith("Custom_Cijk"):
            name = "hipBLASLt " + ("Custom_" if name.startswith("Custom") else "") + name.split("_MT")[1].split("_")[0]
        k = (name, int(r["Grid_Size"]) // int(r["Workgroup_Size"]))
        d[k][r["Counter_Name"]].append((float(r["Counter_Value"]),
                                        (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    lines = [f"# Clock and MFMA activity: {tag}", "",
             "Command (from the repository root, on one MI355X):", "", "```", CLOCK_CMD, "```", "",
             "GRBM_GUI_ACTIVE is reported summed over the 8 XCD instances, so cycles per instance are "
             "the value / 8. MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles per instance x 1024 SIMDs). "
             "The apparent clock (cycles per instance / duration) includes a fixed per-dispatch "
             "overhead of a few thousand cycles, which inflates it for short kernels; the long GEMM "
             "launches below are the meaningful rows. The `hipBLASLt` rows are the library's dense bf16 "
             "GEMM that bench.py times on the same shapes (its `context` field).", "",
             "| kernel | grid WGs | dispatches | avg us | cycles per XCD | apparent clock GHz | MFMA busy % |",
             "|---|---|---|---|---|---|---|"]
    keep = [k for k in d if k[0].startswith("qlora_gemm") or k[0].startswith("hipBLASLt")]
    for k in sorted(keep, key=lambda k: (k[0], k[1])):
        g = d[k]["GRBM_GUI_ACTIVE"]
        mf = d[k]["SQ_VALU_MFMA_BUSY_CYCLES"]
        cyc = sum(x for x, _ in g) / len(g) / 8
        dur = sum(t for _, t in g) / len(g)
        mfb = sum(x for x, _ in mf) / len(mf) if mf else 0.0
        lines.append(f"| `{k[0]}` | {k[1]} | {len(g)} | {dur:.1f} | {cyc:.0f} | {cyc/dur/1e3:.2f} | "
                     f"{100*mfb/(cyc*1024):.1f} |")
    # the same kernel at two launch sizes gives the clock without the fixed overhead
    a = d.get(("qlora_gemm_kernel<false, 256, false>", 256)); b = d.get(("qlora_gemm_kernel<false, 256, false>", 896))
    if a and b:
        ca = sum(x for x, _ in a["GRBM_GUI_ACTIVE"]) / len(a["GRBM_GUI_ACTIVE"]) / 8
        ta = sum(t for _, t in a["GRBM_GUI_ACTIVE"]) / len(a["GRBM_GUI_ACTIVE"])
        cb = sum(x for x, _ in b["GRBM_GUI_ACTIVE"]) / len(b["GRBM_GUI_ACTIVE"]) / 8
        tb = sum(t for _, t in b["GRBM_GUI_ACTIVE"]) / len(b["GRBM_GUI_ACTIVE"])
        slope = (cb - ca) / (tb - ta) / 1e3
        lines += ["", f"Fit over the two launch sizes of `qlora_gemm_kernel<false, 256, false>` (256 and 896 "
                      f"workgroups): {slope:.2f} GHz sustained, {ca - slope*1e3*ta:.0f} cycles of fixed "
                      f"overhead per dispatch.", ""]
    return "\n".join(lines)


LDS_CMD = ("timeout -s KILL 240 rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT "
           "SQ_LDS_DATA_FIFO_FULL SQ_LDS_ADDR_CONFLICT SQ_BUSY_CU_CYCLES SQ_WAIT_INST_LDS SQ_ACTIVE_INST_LDS "
           "--output-format csv -d gpurun_out/pmc_lds -o run -- python3 bench.py --steps 2 --warmup 0 "
           "--no-cpu-baseline --no-paths")


def lds(tag):
    rows = list(csv.DictReader(open(f"{OUT}/pmc_lds/run_counter_collection.csv")))
    d = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in rows:
        name = short(r["Kernel_Name"])
        if name.startswith("Custom_Cijk"):
            name = "hipBLASLt Custom_" + name.split("_MT")[1].split("_")[0]
        elif name.startswith("Cijk"):
            name = "hipBLASLt " + name.split("_MT")[1].split("_")[0]
        d[(name, int(r["Grid_Size"]) // int(r["Workgroup_Size"]))][r["Counter_Name"]].append(
            float(r["Counter_Value"]))
    lines = [f"# LDS activity of the fused GEMMs: {tag}", "",
             "Command (from the repository root, on one MI355X):", "", "```", LDS_CMD, "```", "",
             "Per dispatch, averaged over the dispatches of each kernel and grid. GRBM_GUI_ACTIVE is summed "
             "over the 8 XCD instances, so cycles per instance are the value / 8; LDS active = "
             "SQ_LDS_IDX_ACTIVE / (cycles x 256 CUs), and likewise the bank-conflict and data-FIFO-full "
             "stall cycles (the tool's own LDS utilisation and bank-conflict metrics). The `hipBLASLt` "
             "rows are the library's dense bf16 GEMM that bench.py times on the same shapes.", "",
             "| kernel | grid WGs | dispatches | cycles per XCD | LDS active % | bank-conflict stall % | "
             "data FIFO full % |", "|---|---|---|---|---|---|---|"]
    for k in sorted(d):
        if not (k[0].startswith("qlora_gemm") or k[0].startswith("hipBLASLt")):
            continue
        c = {n: sum(v) / len(v) for n, v in d[k].items()}
        g = c["GRBM_GUI_ACTIVE"] / 8
        lines.append(f"| `{k[0]}` | {k[1]} | {len(d[k]['GRBM_GUI_ACTIVE'])} | {g:.0f} | "
                     f"{100 * c['SQ_LDS_IDX_ACTIVE'] / (g * 256):.1f} | "
                     f"{100 * c['SQ_LDS_BANK_CONFLICT'] / (g * 256):.1f} | "
                     f"{100 * c['SQ_LDS_DATA_FIFO_FULL'] / (g * 256):.1f} |")
    lines.append("")
    return "\n".join(lines)


if __name__ == "__main__":
    tag = sys.argv[1]
    bench_json = f"{OUT}/bench.json"
    os.makedirs(PROF, exist_ok=True)
    open(f"{PROF}/fused_gemm_llama8b_kernel_trace.md", "w").write(ktrace(tag, bench_json))
    text, traffic = counters(tag, bench_json)
    open(f"{PROF}/fused_gemm_llama8b_hbm_counters.md", "w").write(text)
    json.dump(traffic, open(f"{PROF}/traffic.json", "w"), indent=1)
    line = open(bench_json).read().strip()
    open(f"{PROF}/bench_llama8b.md", "w").write(
        f"# Benchmark line: {tag}\n\nCommand (from the repository root, on one MI355X):\n\n```\n"
        f"python3 bench.py\n```\n\nOutput:\n\n```\n{line}\n```\n")
    if os.path.exists(f"{OUT}/ktrace_paths/run_kernel_stats.csv"):
        open(f"{PROF}/bandwidth_paths_kernel_trace.md", "w").write(paths_trace(tag))
        print(open(f"{PROF}/bandwidth_paths_kernel_trace.md").read())
    if os.path.exists(f"{OUT}/pmc_lds/run_counter_collection.csv"):
        open(f"{PROF}/fused_gemm_llama8b_lds_counters.md", "w").write(lds(tag))
        print(open(f"{PROF}/fused_gemm_llama8b_lds_counters.md").read())
    if os.path.exists(f"{OUT}/pmc_clock/run_counter_collection.csv"):
        open(f"{PROF}/fused_gemm_llama8b_clock_mfma.md", "w").write(clock(tag))
        print(open(f"{PROF}/fused_gemm_llama8b_clock_mfma.md").read())
    print(open(f"{PROF}/fused_gemm_llama8b_kernel_trace.md").read()[:3000])
    print(text)
