#!/usr/bin/env python3
"""Benchmark of the W4A8 / W4A16 hot path on one MI355X.

Headline workload: W4A8 int8 per-channel GEMM at N=8192, K=21760 (the GEMM
shape the W4A8 Marlin PR benchmarks), M in {1, 16, 64, 256, 1024, 4096}.  One
step is one pass of the per-call path over every M: dynamic per-token int8
quantisation of fp16 activations [M, K], then the W4A8 GEMM with int4 weights
(prepacked once, PB-v1) and fp32 per-channel scales, fp16 output.  All inputs
are seeded synthetic data resident in HBM before timing starts; each M reads
its own weight copy, so consecutive launches never find their weight in the
256 MB last-level cache.

The line also carries every other workload of the method at each of its M
(``configs``): the M=16 N=256 K=512 per-channel problem, the W4A16 bf16
group-128 decode GEMM 4096 x 4096, the int8 group-128 7B-style decoder-layer
shapes and the fp8 group-128 GEMM 28672 x 8192.  Each point is timed over
back-to-back launches that rotate through at least 512 MB of weight copies,
and is set against its roofline (HBM below the ridge, the MFMA peak of its
operand type above it).  These launches are captured in a HIP graph and
replayed, so that the host's launch rate does not bound the short ones.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints one JSON line.  value = total GEMM ops of a headline step (2*M*N*K
summed over the M sweep) / step time, in TOPS (int8).  Also: per-M timings,
the roofline of the dominant kernel, the prepack (a load-time step) and the
CPU oracle timed on a bounded sample as a baseline.

Profiling modes (rocprofv3 runs; see profiles/):

    python bench.py --only SET            # only that set's GEMMs, a few launches each
    python bench.py --summarize SET TRACE_DIR FETCH_DIR WRITE_DIR
    python bench.py --summarize-counters SET DIR [DIR ...]
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

N, K = 8192, 21760
MS = (1, 16, 64, 256, 1024, 4096)
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
PEAK_TOPS = {"i8": 5000.0, "fp8": 5000.0, "f16": 2500.0, "bf16": 2500.0}   # dense MFMA
INT8_PEAK_TOPS = PEAK_TOPS["i8"]
METRIC = "W4A8 GEMM TOPS + weight GB/s (% roofline), N=8192 K=21760, M=1..4096"
CALIB_BYTES = 256 << 20          # plain copy of known size: reads and writes this many bytes
POOL_BYTES = 512 << 20           # weight copies rotated per workload: twice the last-level cache
GEMM_SOURCES = ["mixed_precision_quantized_prepack_amd/csrc/w4_gemm.hip",
                "mixed_precision_quantized_prepack_amd/csrc/w4_gemm_stream.hip",
                "mixed_precision_quantized_prepack_amd/csrc/w4_gemm_pingpong.hip",
                "mixed_precision_quantized_prepack_amd/csrc/w4_gemm_common.h",
                "mixed_precision_quantized_prepack_amd/csrc/w4_device.h",
                "mixed_precision_quantized_prepack_amd/csrc/w4_api.cpp"]

# The method's workloads: (config number, workload name, M values).  A profile
# set groups the workloads one rocprofv3 run covers.
CONFIGS = [
    (1, "w4a8_i8_pc_256x512", (16,)),
    (2, "w4a16_bf16_g128_4096x4096", (1, 4, 16)),
    (3, "w4a8_i8_pc_8192x21760", MS),
    (4, "w4a8_i8_g128_qkv", (1, 16, 128, 1024)),
    (4, "w4a8_i8_g128_o", (1, 16, 128, 1024)),
    (4, "w4a8_i8_g128_gateup", (1, 16, 128, 1024)),
    (4, "w4a8_i8_g128_down", (1, 16, 128, 1024)),
    (5, "w4a8_fp8_g128_28672x8192", (1, 32, 512, 8192)),
]
PROFILE_SETS = {
    "w4a8_i8_pc_8192x21760": ["w4a8_i8_pc_8192x21760"],
    "w4a8_i8_pc_256x512": ["w4a8_i8_pc_256x512"],
    "w4a16_bf16_g128_4096x4096": ["w4a16_bf16_g128_4096x4096"],
    "w4a8_i8_g128_7b_layers": ["w4a8_i8_g128_qkv", "w4a8_i8_g128_o", "w4a8_i8_g128_gateup", "w4a8_i8_g128_down"],
    "w4a8_fp8_g128_28672x8192": ["w4a8_fp8_g128_28672x8192"],
}


def profile_md(set_name: str, kind: str) -> str:
    return os.path.join(ROOT, "profiles", f"{set_name}_{kind}.md")


def sources_sha256() -> str:
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


# ---------------------------------------------------------------------------
# Algorithmic work of one launch.
# ---------------------------------------------------------------------------
def op_name(wl) -> str:
    return wl.q_dtype if wl.kind == "w4a8" else wl.a_dtype


def kernel_label(plan, wl) -> str:
    path, split, tm, tn = plan
    grp = "per-channel" if wl.group_size == wl.K else f"g{wl.group_size}"
    op = {"i8": "int8", "fp8": "fp8", "f16": "fp16", "bf16": "bf16"}[op_name(wl)]
    if path == 1:
        return f"w4_gemm_skinny<{op}, {grp}, {tn // 16} strip(s)>"
    kern = {3: "w4_gemm_stream", 4: "w4_gemm_pingpong"}.get(path, "w4_gemm_tiled")
    return f"{kern}<{op}, {grp}, {tm}x{tn} tile, {'K split' if split > 1 else 'no K split'}>"


def gemm_alg_bytes(wl, M: int, n: int = None, k: int = None) -> int:
    """Packed weight + weight scales (+ zero-points) + activations (+ their
    scales) + output, each once."""
    n = wl.N if n is None else n
    k = wl.K if k is None else k
    sb = {"f32": 4, "f16": 2, "bf16": 2}[wl.s_dtype]
    groups = 1 if wl.group_size == wl.K else k // wl.group_size
    scales = n * groups * sb * (2 if wl.has_zeros else 1)
    act = M * k + 4 * M if wl.kind == "w4a8" else 2 * M * k
    return n * k // 2 + scales + act + 2 * M * n


def roofline_point(wl, M: int, us: float) -> dict:
    """Bound (HBM below the ridge, MFMA above), fraction of that peak, and
    the time the targets ask for (70% of HBM, 50% of MFMA)."""
    ops = 2.0 * M * wl.N * wl.K
    nbytes = gemm_alg_bytes(wl, M)
    peak = PEAK_TOPS[op_name(wl)]
    t_hbm = nbytes / (HBM_PEAK_GBPS * 1e9) * 1e6
    t_mma = ops / (peak * 1e12) * 1e6
    hbm = t_hbm >= t_mma
    frac = (t_hbm if hbm else t_mma) / us
    return {"bound": "hbm" if hbm else "mfma", "frac": round(frac, 4),
            "target_us": round(t_hbm / 0.7 if hbm else t_mma / 0.5, 2),
            "tops": round(ops / (us * 1e-6) / 1e12, 2), "weight_GBps": round(wl.N * wl.K / 2 / (us * 1e-6) / 1e9, 1),
            "alg_GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}


def quant_alg_bytes(M: int) -> int:
    return 2 * M * K + M * K + 4 * M


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands.
# ---------------------------------------------------------------------------
def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(seconds: float) -> dict:
    """The oracle (numpy, float64 matrix products) on a bounded sample of the
    headline workload: 64 rows x 1024 output columns at the full K, on every
    host thread BLAS uses, then 16 rows x 256 columns on one thread."""
    import numpy as np
    import threadpoolctl

    import workloads
    from oracle import w4_oracle as O
    wl = workloads.WORKLOADS["w4a8_i8_pc_8192x21760"]

    def run(Ms, Ns, secs):
        case = workloads.make_case(wl, Ms, N=Ns, K=K, seed_base=42)
        ab = case.a.view(__import__("torch").int16).numpy().view(np.uint16)
        wl_np = case.w_logical.numpy()
        s = case.w_scales.numpy()
        iters, t0 = 0, time.perf_counter()
        while True:
            codes, sa = O.quant_act_per_token(ab, "f16", "i8")
            O.w4a8_gemm(codes, "i8", sa, wl_np, K, "int4", s, "f32", K, "f16")
            iters += 1
            el = time.perf_counter() - t0
            if el >= secs:
                return 2.0 * Ms * Ns * K * iters / el / 1e12, iters, el

    info = threadpoolctl.threadpool_info()
    blas = [i for i in info if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    lib = f"{blas[0].get('internal_api', '?')} {blas[0].get('version', '?')}" if blas else "unknown BLAS"
    v, iters, el = run(64, 1024, seconds)
    with threadpoolctl.threadpool_limits(1):
        v1, iters1, el1 = run(16, 256, max(2.0, seconds / 4))
    return {"value": round(v, 6), "unit": "TOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"M=64 rows x N=1024 columns x K={K} (int8 per-token quant + exact int4 GEMM + fp64 "
                      f"epilogue), {iters} runs in {el:.1f} s on {threads} threads; host has {os.cpu_count()} CPUs",
            "cpu_model": _cpu_model(),
            "implementation": f"numpy {np.__version__} float64 matrix products ({lib}); Python 3 "
                              f"{sys.version.split()[0]}; no compiler flags (interpreted + prebuilt BLAS)",
            "value_1_thread": round(v1, 6),
            "sample_1_thread": f"M=16 rows x N=256 columns x K={K}, {iters1} runs in {el1:.1f} s on one thread"}


# ---------------------------------------------------------------------------
# rocprofv3 summaries.
# ---------------------------------------------------------------------------
def _read_csv(d: str, suffix: str):
    files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _short(name: str) -> str:
    return re.sub(r"\s+", " ", name.split("(")[0].replace("void ", ""))


def _dispatch_counters(d: str, counter: str):
    """{(kernel, grid): [value per dispatch]} for one counter."""
    out = {}
    for r in _read_csv(d, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        key = (_short(r["Kernel_Name"]), int(float(r.get("Grid_Size", 0) or 0)))
        out.setdefault(key, []).append(float(r["Counter_Value"]))
    return out


def _profile_cmds(set_name: str, trace_dir: str, fetch_dir: str, write_dir: str):
    base = f"python -u bench.py --only {set_name} --calibrate-copy"
    return [f"rocprofv3 --kernel-trace --stats --output-format csv -d {trace_dir} -o trace -- {base}",
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o fetch -- {base}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o write -- {base}",
            f"python bench.py --summarize {set_name} {trace_dir} {fetch_dir} {write_dir}"]


def summarize(set_name: str, trace_dir: str, fetch_dir: str, write_dir: str) -> int:
    fetch = _dispatch_counters(fetch_dir, "FETCH_SIZE")
    write = _dispatch_counters(write_dir, "WRITE_SIZE")
    calib_f = [v for (k, g), vs in fetch.items() if "bitwise_not" in k.lower() for v in vs]
    calib_w = [v for (k, g), vs in write.items() if "bitwise_not" in k.lower() for v in vs]
    f_factor = CALIB_BYTES / (1024 * (sum(calib_f) / len(calib_f))) if calib_f else None
    w_factor = CALIB_BYTES / (1024 * (sum(calib_w) / len(calib_w))) if calib_w else None
    kernels = {}
    for (k, g), vs in fetch.items():
        if not k.startswith("w4::"):
            continue
        wv = write.get((k, g), [])
        kernels[f"{k} grid={g}"] = {
            "dispatches": len(vs), "fetch_KiB_avg": sum(vs) / len(vs),
            "write_KiB_avg": (sum(wv) / len(wv)) if wv else None,
            "hbm_bytes_per_launch": (sum(vs) / len(vs) * 1024 * f_factor +
                                     ((sum(wv) / len(wv)) * 1024 * w_factor if wv else 0.0))
            if f_factor and w_factor else None}
    data = {"source_sha256": sources_sha256(), "fetch_factor": f_factor, "write_factor": w_factor,
            "kernels": kernels}
    cmds = _profile_cmds(set_name, trace_dir, fetch_dir, write_dir)
    lines = [f"# HBM traffic: {set_name} ({', '.join(PROFILE_SETS[set_name])})", "",
             "Commands (repository root, one MI355X; each counter in its own run):", "", "```", *cmds, "```", "",
             "FETCH_SIZE / WRITE_SIZE are KiB per dispatch.  They are scaled by what the same counters read "
             f"for a plain copy kernel that reads and writes {CALIB_BYTES >> 20} MiB "
             f"(fetch factor {f_factor if f_factor is None else round(f_factor, 4)}, "
             f"write factor {w_factor if w_factor is None else round(w_factor, 4)}).  Grids are in threads; "
             "each GEMM point has its own grid unless two M share one.", "",
             "| kernel | grid | dispatches | FETCH KiB | WRITE KiB | HBM bytes / launch |", "|---|---|---|---|---|---|"]
    for name, v in sorted(kernels.items()):
        k, g = name.rsplit(" grid=", 1)
        lines.append(f"| `{k[:100]}` | {g} | {v['dispatches']} | {v['fetch_KiB_avg']:.0f} | "
                     f"{v['write_KiB_avg'] if v['write_KiB_avg'] is None else round(v['write_KiB_avg'])} | "
                     f"{v['hbm_bytes_per_launch'] if v['hbm_bytes_per_launch'] is None else int(v['hbm_bytes_per_launch'])} |")
    lines += ["", "Machine-readable (read by bench.py while the GEMM sources hash the same):", "", "```json",
              json.dumps(data, indent=1), "```", ""]
    path = profile_md(set_name, "hbm_traffic")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        fh.write("\n".join(lines))
    print(path)
    write_kernel_stats(set_name, trace_dir, cmds[0])
    return 0


STEP_PROFILE_ARGS = "--no-configs --no-cpu-baseline"


def summarize_step(trace_dir: str) -> int:
    """Kernel-time summary of a trace of the headline step itself (the timed
    steps and the per-launch event pass of the default run, without the
    workload sweep): the figures the bench line's roofline is taken from."""
    cmd = (f"rocprofv3 --kernel-trace --stats --output-format csv -d {trace_dir} -o trace -- "
           f"python -u bench.py {STEP_PROFILE_ARGS}")
    write_kernel_stats("w4a8_i8_pc_8192x21760", trace_dir, cmd, kind="step_kernel_stats",
                       what="the headline step (per-token quantisation and GEMM at M = 1 ... 4096, "
                            "settle, warm-up, timed steps and the per-launch event pass)")
    return 0


def write_kernel_stats(set_name: str, trace_dir: str, cmd: str, kind: str = "kernel_stats",
                       what: str = "") -> None:
    """Kernel-time summary of the trace run (rocprofv3 --kernel-trace --stats)."""
    rows = sorted(_read_csv(trace_dir, "kernel_stats.csv"), key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# Kernel statistics: {set_name} ({what or ', '.join(PROFILE_SETS[set_name])})", "",
             "Command (repository root, one MI355X):", "", "```", cmd, "```", "",
             "Durations are per dispatch, from the kernel trace.", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{_short(r['Name'])[:110]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.2f} |")
    per_grid = {}
    for r in _read_csv(trace_dir, "kernel_trace.csv"):
        k = _short(r["Kernel_Name"])
        if not k.startswith("w4::w4_gemm") and not k.startswith("w4::w4_splitk"):
            continue
        key = (k, int(float(r.get("Grid_Size_X", r.get("Grid_Size", 0)) or 0)))
        per_grid.setdefault(key, []).append(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]))))
    lines += ["", "GEMM launches by grid (threads); the last column lists the last eight launches in launch order:",
              "", "| kernel | grid | calls | avg us | median us | last launches us |", "|---|---|---|---|---|---|"]
    for (k, g), v in sorted(per_grid.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        d = [(e - b) / 1e3 for b, e in sorted(v)]
        med = sorted(d)[len(d) // 2]
        shown = ("..., " if len(d) > 8 else "") + ", ".join(f"{x:.1f}" for x in d[-8:])
        lines.append(f"| `{k[:110]}` | {g} | {len(d)} | {sum(d) / len(d):.1f} | {med:.1f} | {shown} |")
    path = profile_md(set_name, kind)
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(path)


XCDS = 8          # MI355X: GRBM_GUI_ACTIVE sums the busy cycles of the 8 XCDs
SIMDS = 1024      # 256 CUs x 4 SIMDs


def summarize_counters(set_name: str, dirs) -> int:
    """MFMA / VALU / wait / L2 counters per GEMM dispatch (each directory one
    rocprofv3 --pmc run over the same launches) -> profiles/<set>_mfma_counters.md."""
    per = {}
    for d in dirs:
        for r in _read_csv(d, "counter_collection.csv"):
            k = _short(r["Kernel_Name"])
            if not k.startswith("w4::w4_gemm"):
                continue
            key = (k, int(float(r.get("Grid_Size", 0) or 0)))
            c = per.setdefault(key, {})
            c.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            c.setdefault("_dur_" + os.path.basename(d.rstrip("/")), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"# MFMA, VALU, wait and L2 counters: {set_name} ({', '.join(PROFILE_SETS[set_name])})", "",
             "Commands (repository root, one MI355X; one counter group per run, each over the same launches):", "",
             "```"]
    lines += [f"rocprofv3 --pmc <group> --output-format csv -d {d} -o pmc -- python -u bench.py --only {set_name}"
              for d in dirs]
    lines += [f"python bench.py --summarize-counters {set_name} {' '.join(dirs)}", "```", "",
              "Groups: SQ_INSTS_VALU_MFMA_MOPS_I8 SQ_INSTS_VALU_MFMA_MOPS_F8 SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU "
              "SQ_INSTS_MFMA SQ_BUSY_CYCLES SQ_WAVE_CYCLES GRBM_GUI_ACTIVE | SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU "
              "SQ_ACTIVE_INST_LDS SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_VMEM SQ_WAVES SQ_CYCLES | "
              "TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_DRAM_sum.", "",
              f"Derived, averaged over the dispatches of each kernel and grid (threads): clock = GRBM_GUI_ACTIVE / "
              f"({XCDS} XCDs x duration); MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / ({SIMDS} SIMDs x GRBM_GUI_ACTIVE / "
              f"{XCDS}); MFMA ops = 512 x SQ_INSTS_VALU_MFMA_MOPS_(I8 + F8) (equal to 2 M N K when the tile covers "
              "M and N exactly); VALU / MFMA = SQ_INSTS_VALU / SQ_INSTS_MFMA; wait = SQ_WAIT_INST_ANY / "
              "SQ_WAVE_CYCLES (share of resident wave cycles in which the wave had an instruction waiting to issue: on a dependency, a wait count or a unit busy with another wave); the clock and MFMA busy "
              "columns hold for launches of ~50 us or more (GRBM_GUI_ACTIVE also counts cycles outside a short "
              "kernel's own timestamps); L2 hit = TCC_HIT / (TCC_HIT + "
              "TCC_MISS); EA reads = TCC_EA0_RDREQ (requests from the L2s to the fabric, each 64 B or 128 B; "
              "TCC_EA0_RDREQ_DRAM counts the same requests, Infinity Cache hits included, so the counters do not "
              "separate Infinity Cache hits from HBM reads).", "",
              "| kernel | grid | us | clock GHz | MFMA busy | MFMA Gops | VALU / MFMA | wait | LDS bank conflicts / LDS instr | "
              "L2 hit | EA read req | EA DRAM req |", "|---|---|---|---|---|---|---|---|---|---|---|---|"]

    def avg(c, n):
        v = c.get(n)
        return sum(v) / len(v) if v else None
    for (k, g), c in sorted(per.items()):
        durs = [avg(c, n) for n in c if n.startswith("_dur_")]
        dur = min(durs) if durs else None
        gui = avg(c, "GRBM_GUI_ACTIVE")
        clk = gui / XCDS / (dur * 1e3) if gui and dur else None
        busy = avg(c, "SQ_VALU_MFMA_BUSY_CYCLES")
        busy = busy / (SIMDS * gui / XCDS) if busy is not None and gui else None
        mops = (avg(c, "SQ_INSTS_VALU_MFMA_MOPS_I8") or 0.0) + (avg(c, "SQ_INSTS_VALU_MFMA_MOPS_F8") or 0.0)
        valu, mf = avg(c, "SQ_INSTS_VALU"), avg(c, "SQ_INSTS_MFMA")
        wait, wcyc = avg(c, "SQ_WAIT_INST_ANY"), avg(c, "SQ_WAVE_CYCLES")
        hit, miss = avg(c, "TCC_HIT_sum"), avg(c, "TCC_MISS_sum")
        bc, lds = avg(c, "SQ_LDS_BANK_CONFLICT"), avg(c, "SQ_INSTS_LDS")
        f = lambda v, fmt: "" if v is None else format(v, fmt)  # noqa: E731
        lines.append(
            f"| `{k[:100]}` | {g} | {f(dur, '.1f')} | {f(clk, '.2f')} | {f(busy, '.3f')} | {mops * 512 / 1e9:.1f} | "
            f"{f(valu / mf if valu and mf else None, '.2f')} | {f(wait / wcyc if wait and wcyc else None, '.3f')} | "
            f"{f(bc / lds if bc is not None and lds else None, '.3f')} | "
            f"{f(hit / (hit + miss) if hit is not None and miss is not None and hit + miss else None, '.3f')} | "
            f"{f(avg(c, 'TCC_EA0_RDREQ_sum'), '.3g')} | {f(avg(c, 'TCC_EA0_RDREQ_DRAM_sum'), '.3g')} |")
    path = profile_md(set_name, "mfma_counters")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(path)
    return 0


def traffic_for(set_name: str, kernel_key: str, grids) -> "float | None":
    """HBM bytes per launch of a kernel from the committed counter summary of
    its set, or None if there is none or the GEMM sources changed since."""
    try:
        with open(profile_md(set_name, "hbm_traffic")) as fh:
            text = fh.read()
        data = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None
    if data.get("source_sha256") != sources_sha256():
        return None
    vals = [v["hbm_bytes_per_launch"] for k, v in data["kernels"].items()
            if v.get("hbm_bytes_per_launch") and k.startswith(kernel_key + " ")
            and int(k.rsplit("grid=", 1)[1]) in grids]
    return round(sum(vals) / len(vals)) if vals else None


def kernel_key_of(wl, plan, M: int) -> str:
    """The kernel trace's name of the GEMM instance a plan launches at M."""
    path, split, tm, tn = plan
    op = {"i8": 0, "fp8": 1, "f16": 2, "bf16": 3}[op_name(wl)]
    grouped = "true" if wl.group_size != wl.K else "false"
    if path == 1:
        # 8-bit activations are staged in LDS from M = 8 (the last flag)
        staged = "true" if op in (0, 1) and M >= 8 else "false"
        return f"w4::w4_gemm_skinny<{op}, {grouped}, false, {tn // 16}, false, false, 1, false, false, {staged}>"
    nt, mt = tn // 64, tm // 16
    if path == 4:
        # 128-row tiles are the form whose two halves split K
        return (f"w4::w4_gemm_pingpong<{'true' if tm == 128 else 'false'}, false, "
                f"{'true' if split > 1 else 'false'}, false>")
    if path == 3:
        stages = min(8, (120 * 1024) // (mt * 16 * 128 + 4 * nt * 1024))
        return (f"w4::w4_gemm_stream<{op}, {grouped}, false, {nt}, {mt}, {stages}, "
                f"{'true' if split > 1 else 'false'}, false>")
    return (f"w4::w4_gemm_tiled<{op}, {grouped}, false, {nt}, {mt}, {'true' if split > 1 else 'false'}, false, "
            f"false, 1, false>")


def grid_threads(wl, plan, M: int) -> int:
    """Threads of the GEMM launch (the trace's Grid_Size)."""
    path, split, tm, tn = plan
    if path == 1:
        # one workgroup per tn columns, 64 max(S, 4 strips) threads
        return (wl.N // tn) * 64 * max(split, 4 * (tn // 16))
    threads = 512 if path == 4 else 256   # the ping-pong kernel: eight waves
    return ((M + tm - 1) // tm) * ((wl.N + tn - 1) // tn) * split * threads


# ---------------------------------------------------------------------------
# The per-workload sweep.
# ---------------------------------------------------------------------------
class WorkloadBench:
    """Inputs of one workload resident on the device: activations for the
    largest M, a pool of weight copies of at least POOL_BYTES, scales,
    zero-points, per-M quantised activations and outputs."""

    def __init__(self, wl, Ms, dev, seed=2024):
        import torch

        import mixed_precision_quantized_prepack_amd as w4
        import workloads
        self.torch, self.w4, self.wl, self.Ms = torch, w4, wl, Ms
        case = workloads.make_case(wl, max(Ms), seed_base=seed)
        self.a = case.a.to(dev)
        self.scales = case.w_scales.to(dev)
        self.zeros = None if case.zeros is None else case.zeros.to(dev)
        operand = "i8" if wl.kind == "w4a8" else "f16"
        w0 = w4.prepack_B(case.w_logical.to(dev), operand)
        wbytes = wl.N * wl.K // 2
        self.copies = max(2, min(64, math.ceil(POOL_BYTES / wbytes)))
        # XOR with a per-copy byte: a bijection on each 4-bit code, so every
        # copy is a valid weight of the same distribution
        self.packed = [w0] + [w0 ^ ((i * 0x37 + 0x5A) & 0xFF) for i in range(1, self.copies)]
        self.gs = -1 if wl.group_size == wl.K else wl.group_size
        self.out_dt = torch.float16 if wl.out_dtype == "f16" else torch.bfloat16
        self.a_code = {"i8": w4.I8, "fp8": w4.FP8_E4M3, "f16": w4.F16, "bf16": w4.BF16}[op_name(wl)]
        self.aq, self.sa, self.out = {}, {}, {}
        for M in Ms:
            self.out[M] = torch.empty((M, wl.N), dtype=self.out_dt, device=dev)
            if wl.kind == "w4a8":
                self.aq[M], self.sa[M] = w4.quant_act_per_token(self.a[:M].contiguous(), wl.q_dtype)
        ws = max(w4.gemm_workspace_bytes(M, wl.N, wl.K, self.gs, self.a_code) for M in Ms)
        self.ws = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
        self.plans = {M: w4.gemm_plan(M, wl.N, wl.K, self.gs, self.a_code) for M in Ms}
        self.a_rows = {M: self.a[:M].contiguous() for M in Ms}

    def gemm(self, M: int, r: int):
        w4, wl = self.w4, self.wl
        b = self.packed[r % self.copies]
        if wl.kind == "w4a8":
            w4.w4a8_gemm(self.aq[M], self.sa[M], b, self.scales, self.gs, self.out_dt, out=self.out[M],
                         workspace=self.ws)
        else:
            w4.w4a16_gemm(self.a_rows[M], b, self.scales, self.zeros, self.gs, out=self.out[M], workspace=self.ws)

    def quant(self, M: int):
        self.w4.quant_act_per_token(self.a_rows[M], self.wl.q_dtype, out=self.aq[M], scales=self.sa[M])

    def time_us(self, fn, reps: int, replays: int = 3) -> float:
        """Average launch time of `reps` launches captured in one HIP graph
        (so that the host's launch rate, ~8 us per call from Python, does not
        bound short kernels), over the fastest of `replays` replays timed with
        events on the launch stream."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(reps):
                fn(r + 1)
        g.replay()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(replays):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3 / reps)
        del g
        return best

    def sweep(self, config: int, min_ms: float = 10.0) -> list:
        wl = self.wl
        rows = []
        for M in self.Ms:
            # a first estimate sizes the captured batch: at least 20 launches
            # and about min_ms of GPU time per replay
            est = self.time_us(lambda r: self.gemm(M, r), 3, 1)
            reps = int(max(20, min(200, min_ms * 1e3 / max(est, 1.0))))
            us = self.time_us(lambda r: self.gemm(M, r), reps)
            row = {"config": config, "workload": wl.name, "M": M, "N": wl.N, "K": wl.K,
                   "kernel": kernel_label(self.plans[M], wl), "k_split": self.plans[M][1],
                   "gemm_us": round(us, 2), "launches": reps, "timing": "graph replay, fastest of 3",
                   "weight_copies": self.copies}
            row.update(roofline_point(wl, M, us))
            row["meets_target"] = us <= row["target_us"]
            if wl.kind == "w4a8":
                row["quant_us"] = round(self.time_us(lambda r: self.quant(M), 20), 2)
            rows.append(row)
        return rows


def run_only(set_name: str, calibrate: bool) -> int:
    """A short run of one profile set's GEMMs for rocprofv3: a few launches
    per M (rotating weight copies) after a short warm-up."""
    import torch

    import mixed_precision_quantized_prepack_amd as w4
    import workloads
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w4.lib()
    if calibrate:
        calibration_copy(dev)
    for name in PROFILE_SETS[set_name]:
        Ms = next(m for c, n, m in CONFIGS if n == name)
        wb = WorkloadBench(workloads.WORKLOADS[name], Ms, dev)
        for M in Ms:
            for r in range(8):
                wb.gemm(M, r)
            if wb.wl.kind == "w4a8":
                wb.quant(M)
        torch.cuda.synchronize()
        print(f"profiled {name}: M {list(Ms)}", flush=True)
        del wb
    return 0


def calibration_copy(dev) -> dict:
    """A plain 256 MiB device copy (read + write), for scaling HBM counters."""
    import torch
    src = torch.zeros(CALIB_BYTES // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    ce = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.bitwise_not(src, out=dst)                  # warm-up
    ce[0].record()
    torch.bitwise_not(src, out=dst)                  # plain copy kernel: reads and writes 256 MiB
    ce[1].record()
    torch.cuda.synchronize()
    us = ce[0].elapsed_time(ce[1]) * 1e3
    return {"bytes_read": CALIB_BYTES, "bytes_written": CALIB_BYTES, "us": round(us, 2),
            "GBps_read_plus_write": round(2 * CALIB_BYTES / (us * 1e-6) / 1e9, 1)}


# ---------------------------------------------------------------------------
# Main benchmark.
# ---------------------------------------------------------------------------
def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed steps for at least this long before the warm-up steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the sweep over the other workloads")
    ap.add_argument("--ms", default=",".join(str(m) for m in MS))
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (read + write) to scale HBM counters")
    ap.add_argument("--only", choices=sorted(PROFILE_SETS), help="only this set's GEMMs (for rocprofv3)")
    ap.add_argument("--summarize", nargs=4, metavar=("SET", "TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the kernel-time and HBM-traffic summaries from rocprofv3 outputs and exit")
    ap.add_argument("--summarize-step", metavar="TRACE_DIR",
                    help=f"write the kernel summary of a trace of 'bench.py {STEP_PROFILE_ARGS}' and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="SET_AND_DIRS",
                    help="SET DIR [DIR ...]: write the MFMA/VALU counter summary and exit")
    args = ap.parse_args(argv)
    if args.summarize:
        return summarize(*args.summarize)
    if args.summarize_step:
        return summarize_step(args.summarize_step)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters[0], args.summarize_counters[1:])
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library runs on a single MI355X and has no "
              f"multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2
    if args.only:
        return run_only(args.only, args.calibrate_copy)
    Ms = tuple(int(x) for x in args.ms.split(","))

    import torch

    import mixed_precision_quantized_prepack_amd as w4
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w4.lib()
    wl = workloads.WORKLOADS["w4a8_i8_pc_8192x21760"]

    # ---- inputs, resident in HBM ------------------------------------------
    case = workloads.make_case(wl, max(Ms), seed_base=2024)
    a = case.a.to(dev)
    w0 = case.w_logical.to(dev)
    scales = case.w_scales.to(dev)
    copies = len(Ms)
    logical = [workloads.weight_copy(w0, i).contiguous() for i in range(copies)]
    packed = [torch.empty(N * K // 2, dtype=torch.uint8, device=dev) for _ in range(copies)]
    aq = {M: torch.empty((M, K), dtype=torch.int8, device=dev) for M in Ms}
    sa = {M: torch.empty((M,), dtype=torch.float32, device=dev) for M in Ms}
    out = {M: torch.empty((M, N), dtype=torch.float16, device=dev) for M in Ms}
    ws_bytes = max(w4.gemm_workspace_bytes(M, N, K, -1, w4.I8) for M in Ms)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    plans = {M: w4.gemm_plan(M, N, K, -1, w4.I8) for M in Ms}

    calib = calibration_copy(dev) if args.calibrate_copy else None

    # prepack (load-time): one launch per weight copy, timed with events
    pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(copies)]
    for i in range(copies):
        pev[i][0].record()
        w4.prepack_B(logical[i], "i8", out=packed[i])
        pev[i][1].record()
    torch.cuda.synchronize()
    prepack_us = sorted(s.elapsed_time(e) * 1e3 for s, e in pev)
    del logical
    # import of the same-size weight from ExLlama-shuffled int32 words
    words = torch.randint(-2 ** 31, 2 ** 31 - 1, (N, K // 8), dtype=torch.int32, device=dev)
    scratch = torch.empty(N * K // 2, dtype=torch.uint8, device=dev)
    w4.prepack_B_from_exllama(words, "i8", out=scratch)
    xev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
    for e0, e1 in xev:
        e0.record()
        w4.prepack_B_from_exllama(words, "i8", out=scratch)
        e1.record()
    torch.cuda.synchronize()
    import_us = sorted(a.elapsed_time(b) * 1e3 for a, b in xev)
    del words, scratch

    def step(evs):
        for i, M in enumerate(Ms):
            if evs is not None:
                evs[i][0].record()
            w4.quant_act_per_token(a[:M], "i8", out=aq[M], scales=sa[M])
            if evs is not None:
                evs[i][1].record()
            w4.w4a8_gemm(aq[M], sa[M], packed[i % copies], scales, -1, torch.float16, out=out[M],
                         workspace=ws)
            if evs is not None:
                evs[i][2].record()

    # Clock settle: the GPU raises its clocks over the first tens of ms of
    # sustained work (a step after ~3 ms of warm-up runs ~13% slower than one
    # after 100 ms), so untimed steps run for at least --settle-ms before the
    # W warm-up steps.
    settle_steps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(5):
            step(None)
        settle_steps += 5
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()

    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    all_evs = [[(mk(), mk(), mk()) for _ in Ms] for _ in range(args.steps)]
    t_start, t_end = mk(), mk()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    # The headline: K steps with nothing between the launches.  An event
    # recorded between two kernels costs several us of dispatch latency, so
    # the per-launch durations come from a second pass of K steps with events
    # around every launch on the launch stream.
    t_start.record()
    for s in range(args.steps):
        step(None)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    e_start, e_end = mk(), mk()
    e_start.record()
    for s in range(args.steps):
        step(all_evs[s])
    e_end.record()
    torch.cuda.synchronize()
    ms_per_step_events = e_start.elapsed_time(e_end) / args.steps

    # ---- per-launch durations of the short GEMMs ---------------------------
    # A launch of ~20 us bracketed by two events also counts the event-to-
    # kernel dispatch latency (a few us), so GEMMs shorter than 100 us in the
    # step are timed again alone: REPS launches back to back (rotating the
    # weight copies) between two events on the launch stream.  Longer kernels
    # keep their in-step figure, where that latency is negligible.
    REPS = 30
    iso_us = {}
    for i, M in enumerate(Ms):
        g_us = sum(all_evs[s][i][1].elapsed_time(all_evs[s][i][2]) for s in range(args.steps)) * 1e3 / args.steps
        if g_us >= 100.0:
            continue
        e0, e1 = mk(), mk()
        w4.w4a8_gemm(aq[M], sa[M], packed[i % copies], scales, -1, torch.float16, out=out[M], workspace=ws)
        e0.record()
        for r in range(REPS):
            w4.w4a8_gemm(aq[M], sa[M], packed[(i + r) % copies], scales, -1, torch.float16, out=out[M],
                         workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        iso_us[M] = e0.elapsed_time(e1) * 1e3 / REPS

    # ---- fused RMSNorm + per-token quantisation, next to the plain quantiser
    # (same activations; both read 2 B and write 1 B per element) and the
    # per-tensor quantiser (which reads the activations twice: the codes wait
    # for the whole tensor's maximum), REPS launches back to back between two
    # events
    gamma = workloads.norm_weight(K, "f16", seed=2025).to(dev)
    norm_quant = []
    for M in sorted({min(Ms), max(Ms)}):
        row = {"M": M, "K": K}
        for name, fn in (("quant_us", lambda: w4.quant_act_per_token(a[:M], "i8", out=aq[M], scales=sa[M])),
                         ("rmsnorm_quant_us", lambda: w4.rmsnorm_quant_per_token(a[:M], gamma, 1e-6, "i8",
                                                                                 out=aq[M], scales=sa[M])),
                         ("quant_per_tensor_us", lambda: w4.quant_act_per_tensor(a[:M], "i8", out=aq[M],
                                                                                 scales=sa[M]))):
            fn()
            e0, e1 = mk(), mk()
            e0.record()
            for _ in range(REPS):
                fn()
            e1.record()
            torch.cuda.synchronize()
            row[name] = round(e0.elapsed_time(e1) * 1e3 / REPS, 2)
        nbytes = M * K * 3 + 4 * M + 2 * K
        row["rmsnorm_quant_GBps"] = round(nbytes / (row["rmsnorm_quant_us"] * 1e-6) / 1e9, 1)
        row["hbm_frac"] = round(row["rmsnorm_quant_GBps"] / HBM_PEAK_GBPS, 4)
        norm_quant.append(row)

    # ---- asymmetric W4A8 (zero-points; the same codes read as raw uint4)
    # next to the symmetric GEMM, REPS launches back to back per M
    zeros = torch.randint(0, 16, (N,), generator=torch.Generator().manual_seed(7)).to(torch.float16).to(dev)
    zp_rows = []
    for i, M in enumerate(Ms):
        if M not in (min(Ms), 16, 256, max(Ms)):
            continue
        row = {"M": M}
        for name, fn in (("symmetric_us", lambda r: w4.w4a8_gemm(aq[M], sa[M], packed[r % copies], scales, -1,
                                                                 torch.float16, out=out[M], workspace=ws)),
                         ("zero_point_us", lambda r: w4.w4a8_gemm_zp(aq[M], sa[M], packed[r % copies], scales,
                                                                     zeros, -1, torch.float16, out=out[M],
                                                                     workspace=ws))):
            fn(i)
            e0, e1 = mk(), mk()
            e0.record()
            for r in range(REPS):
                fn(i + r)
            e1.record()
            torch.cuda.synchronize()
            row[name] = round(e0.elapsed_time(e1) * 1e3 / REPS, 2)
        zp_rows.append(row)

    # ---- per-M figures ----------------------------------------------------
    per_m = []
    total_ops = 0.0
    for i, M in enumerate(Ms):
        q_us = sum(all_evs[s][i][0].elapsed_time(all_evs[s][i][1]) for s in range(args.steps)) * 1e3 / args.steps
        g_us = sum(all_evs[s][i][1].elapsed_time(all_evs[s][i][2]) for s in range(args.steps)) * 1e3 / args.steps
        ops = 2.0 * M * N * K
        total_ops += ops
        k_us = iso_us.get(M, g_us)
        rp = roofline_point(wl, M, k_us)
        per_m.append({"M": M, "kernel": kernel_label(plans[M], wl), "k_split": plans[M][1],
                      "gemm_us_in_step": round(g_us, 2), "quant_us_in_step": round(q_us, 2),
                      "gemm_us": round(k_us, 2), "gemm_timing": "back-to-back" if M in iso_us else "in-step",
                      "gemm_tops": rp["tops"], "weight_GBps": rp["weight_GBps"], "alg_GBps": rp["alg_GBps"],
                      "hbm_frac": round(gemm_alg_bytes(wl, M) / (k_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                      "mfma_frac": round(ops / (k_us * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4),
                      "bound": rp["bound"], "frac": rp["frac"], "target_us": rp["target_us"]})
    value = total_ops / (ms_per_step * 1e-3) / 1e12

    # dominant kernel: the kernel (template instance) with the most time in a step
    by_kernel = {}
    for pm in per_m:
        by_kernel.setdefault(pm["kernel"], []).append(pm)
    dom_name, dom = max(by_kernel.items(), key=lambda kv: sum(pm["gemm_us"] for pm in kv[1]))
    flops = sum(2.0 * pm["M"] * N * K for pm in dom) / len(dom)
    dur = sum(pm["gemm_us"] for pm in dom) / len(dom)
    ach = flops / (dur * 1e-6) / 1e12
    dom_plan = plans[dom[0]["M"]]
    roofline = {"bound": "mfma", "achieved": round(ach, 2), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                "frac": round(ach / INT8_PEAK_TOPS, 4),
                "traffic": traffic_for("w4a8_i8_pc_8192x21760", kernel_key_of(wl, dom_plan, dom[0]["M"]),
                                       {grid_threads(wl, plans[pm["M"]], pm["M"]) for pm in dom}),
                "kernel": dom_name, "launches": [pm["M"] for pm in dom], "avg_launch_us": round(dur, 2),
                "alg_ops_per_launch": flops,
                "note": "int8 operations (2 per multiply-add) per second; avg_launch_us from a second pass of "
                        "the timed steps with events around each launch on the launch stream; kernel trace of "
                        "the same step: profiles/w4a8_i8_pc_8192x21760_step_kernel_stats.md"}
    small = [pm for pm in per_m if pm["kernel"].startswith("w4_gemm_skinny")]
    roofline_small = None
    if small:
        b = sum(gemm_alg_bytes(wl, pm["M"]) for pm in small) / len(small)
        dur = sum(pm["gemm_us"] for pm in small) / len(small)
        gb = b / (dur * 1e-6) / 1e9
        # per M, its own instance's counters (M >= 8 stages the activations)
        per = [traffic_for("w4a8_i8_pc_8192x21760", kernel_key_of(wl, plans[pm["M"]], pm["M"]),
                           {grid_threads(wl, plans[pm["M"]], pm["M"])}) for pm in small]
        small_traffic = round(sum(per) / len(per)) if all(t is not None for t in per) else None
        roofline_small = {"bound": "hbm", "achieved": round(gb, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                          "frac": round(gb / HBM_PEAK_GBPS, 4),
                          "traffic": small_traffic,
                          "kernel": small[0]["kernel"], "launches": [pm["M"] for pm in small],
                          "avg_launch_us": round(dur, 2), "alg_bytes_per_launch": b,
                          "note": f"avg_launch_us from {REPS} back-to-back launches per M between two events"}

    # ---- every workload of the method, at each of its M --------------------
    configs = []
    if not args.no_configs:
        del aq, out, ws, packed
        torch.cuda.empty_cache()
        for config, name, cms in CONFIGS:
            wb = WorkloadBench(workloads.WORKLOADS[name], cms, dev)
            configs += wb.sweep(config)
            del wb
            torch.cuda.empty_cache()

    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": "w4a8_i8_pc_8192x21760", "N": N, "K": K, "Ms": list(Ms),
                   "activations": "fp16 ~N(0,1), dynamic per-token int8", "weights": "int4 uniform [-8,7], PB-v1",
                   "scales": "fp32 per channel ~U(0.005,0.02)", "out": "fp16", "weight_copies": copies},
        "weight_GBps_step": round(copies * (N * K / 2) / (ms_per_step * 1e-3) / 1e9, 1),
        "ms_per_step_with_launch_events": round(ms_per_step_events, 4),
        "settle_steps": settle_steps,
        "per_m": per_m,
        "roofline": roofline,
        "roofline_small_m": roofline_small,
        "configs": configs,
        "rmsnorm_quant": norm_quant,
        "w4a8_zero_point": zp_rows,
        "prepack": {"median_us": round(prepack_us[len(prepack_us) // 2], 2),
                    "GBps_read_plus_write": round(N * K / (prepack_us[len(prepack_us) // 2] * 1e-6) / 1e9, 1)},
        "prepack_from_exllama": {"median_us": round(import_us[len(import_us) // 2], 2),
                                 "GBps_read_plus_write": round(N * K / (import_us[len(import_us) // 2] * 1e-6) / 1e9, 1)},
        "wall_s_timed": round(wall, 3),
    }
    if calib:
        line["copy_calibration"] = calib
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
