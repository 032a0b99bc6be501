#!/usr/bin/env python3
"""Benchmark of the W4A8 hot path on one MI355X.

Workload: W4A8 int8 per-channel GEMM at N=8192, K=21760 (the GEMM shape the
W4A8 Marlin PR benchmarks), M in {1, 16, 64, 256, 1024, 4096}.  One step is
one pass of the per-call path over every M: dynamic per-token int8
quantisation of fp16 activations [M, K], then the W4A8 GEMM with int4 weights
(prepacked once, PB-v1) and fp32 per-channel scales, fp16 output.  All inputs
are seeded synthetic data resident in HBM before timing starts; each M reads
its own weight copy, so consecutive launches never find their weight in the
256 MB last-level cache.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints one JSON line.  value = total GEMM ops of a step (2*M*N*K summed over
the M sweep) / step time, in TOPS (int8).  The line also carries per-M
timings, the roofline of the dominant kernel, the prepack (a load-time step)
and the CPU oracle timed on a bounded sample as a baseline.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

N, K = 8192, 21760
MS = (1, 16, 64, 256, 1024, 4096)
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 MFMA
METRIC = "W4A8 GEMM TOPS + weight GB/s (% roofline), N=8192 K=21760, M=1..4096"
CALIB_BYTES = 256 << 20          # plain copy of known size: reads and writes this many bytes
TRAFFIC_MD = os.path.join(ROOT, "profiles", "w4a8_i8_pc_8192x21760_hbm_traffic.md")
STATS_MD = os.path.join(ROOT, "profiles", "w4a8_i8_pc_8192x21760_kernel_stats.md")
GEMM_SOURCES = ["mixed_precision_quantized_prepack_amd/csrc/w4_gemm.hip",
                "mixed_precision_quantized_prepack_amd/csrc/w4_device.h",
                "mixed_precision_quantized_prepack_amd/csrc/w4_api.cpp"]


def sources_sha256() -> str:
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def kernel_label(path: int, split: int, tm: int, tn: int) -> str:
    if path == 1:
        return f"w4_gemm_skinny<int8, per-channel, {tn // 16} strip(s)>"
    return f"w4_gemm_tiled<int8, per-channel, {tm}x{tn} tile, {'K split' if split > 1 else 'no K split'}>"


def gemm_alg_bytes(M: int) -> int:
    """Algorithmic bytes of one W4A8 GEMM launch: packed weight, fp32 channel
    scales, int8 activations + fp32 row scales, fp16 output."""
    return N * K // 2 + 4 * N + M * K + 4 * M + 2 * M * N


def quant_alg_bytes(M: int) -> int:
    return 2 * M * K + M * K + 4 * M


def cpu_baseline(seconds: float) -> dict:
    """The oracle as it stands (numpy, float64 BLAS) on a bounded sample of
    the same workload: 64 rows x 1024 output columns at the full K."""
    import numpy as np
    import threadpoolctl

    import workloads
    from oracle import w4_oracle as O
    wl = workloads.WORKLOADS["w4a8_i8_pc_8192x21760"]
    Ms, Ns = 64, 1024
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
        if el >= seconds:
            break
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    ops = 2.0 * Ms * Ns * K * iters
    return {"value": round(ops / el / 1e12, 6), "unit": "TOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"M={Ms} rows x N={Ns} columns x K={K} (int8 per-token quant + exact int4 GEMM + "
                      f"fp64 epilogue), {iters} runs in {el:.1f} s; host has {os.cpu_count()} CPUs"}


# ---------------------------------------------------------------------------
# HBM traffic from rocprofv3 counters.
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
    """{(kernel, grid): [value per dispatch]} for one counter (KiB per dispatch)."""
    out = {}
    for r in _read_csv(d, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        key = (_short(r["Kernel_Name"]), int(float(r.get("Grid_Size", 0) or 0)))
        out.setdefault(key, []).append(float(r["Counter_Value"]))
    return out


def summarize(trace_dir: str, fetch_dir: str, write_dir: str) -> int:
    fetch = _dispatch_counters(fetch_dir, "FETCH_SIZE")
    write = _dispatch_counters(write_dir, "WRITE_SIZE")
    calib_f = [v for (k, g), vs in fetch.items() if "BitwiseNot" in k or "bitwise_not" in k for v in vs]
    calib_w = [v for (k, g), vs in write.items() if "BitwiseNot" in k or "bitwise_not" in k for v in vs]
    f_factor = CALIB_BYTES / (1024 * (sum(calib_f) / len(calib_f))) if calib_f else None
    w_factor = CALIB_BYTES / (1024 * (sum(calib_w) / len(calib_w))) if calib_w else None
    stats = {_short(r["Name"]): r for r in _read_csv(trace_dir, "kernel_stats.csv")}
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
    lines = ["# HBM traffic: W4A8 int8 per-channel, N=8192 K=21760, M sweep {1,16,64,256,1024,4096}", "",
             "Commands (repository root, one MI355X; each counter in its own run):", "", "```",
             f"rocprofv3 --kernel-trace --stats --output-format csv -d {trace_dir} -o trace -- "
             "python -u bench.py --steps 2 --warmup 1 --no-cpu-baseline --calibrate-copy",
             f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o fetch -- "
             "python -u bench.py --steps 2 --warmup 1 --no-cpu-baseline --calibrate-copy --settle-ms 0",
             f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o write -- "
             "python -u bench.py --steps 2 --warmup 1 --no-cpu-baseline --calibrate-copy --settle-ms 0",
             f"python bench.py --summarize {trace_dir} {fetch_dir} {write_dir}", "```", "",
             "FETCH_SIZE / WRITE_SIZE are KiB per dispatch.  They are scaled by what the same counters read "
             f"for a plain copy kernel that reads and writes {CALIB_BYTES >> 20} MiB "
             f"(fetch factor {f_factor if f_factor is None else round(f_factor, 4)}, "
             f"write factor {w_factor if w_factor is None else round(w_factor, 4)}).", "",
             "| kernel | grid | dispatches | FETCH KiB | WRITE KiB | HBM bytes / launch |", "|---|---|---|---|---|---|"]
    for name, v in sorted(kernels.items()):
        k, g = name.rsplit(" grid=", 1)
        lines.append(f"| `{k[:90]}` | {g} | {v['dispatches']} | {v['fetch_KiB_avg']:.0f} | "
                     f"{v['write_KiB_avg'] if v['write_KiB_avg'] is None else round(v['write_KiB_avg'])} | "
                     f"{v['hbm_bytes_per_launch'] if v['hbm_bytes_per_launch'] is None else int(v['hbm_bytes_per_launch'])} |")
    lines += ["", "Kernel time from the trace run:", "", "| kernel | calls | avg us |", "|---|---|---|"]
    for k, r in stats.items():
        lines.append(f"| `{k[:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} |")
    lines += ["", "Machine-readable (read by bench.py while the GEMM sources hash the same):", "", "```json",
              json.dumps(data, indent=1), "```", ""]
    os.makedirs(os.path.dirname(TRAFFIC_MD), exist_ok=True)
    with open(TRAFFIC_MD, "w") as fh:
        fh.write("\n".join(lines))
    print(TRAFFIC_MD)
    write_kernel_stats(trace_dir)
    return 0


def write_kernel_stats(trace_dir: str) -> None:
    """Kernel-time summary of the trace run (rocprofv3 --kernel-trace --stats)."""
    rows = sorted(_read_csv(trace_dir, "kernel_stats.csv"), key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["# Kernel statistics: W4A8 int8 per-channel, N=8192 K=21760, M sweep {1,16,64,256,1024,4096}", "",
             "Command (repository root, one MI355X):", "", "```",
             f"rocprofv3 --kernel-trace --stats --output-format csv -d {trace_dir} -o trace -- "
             "python -u bench.py --steps 2 --warmup 1 --no-cpu-baseline --calibrate-copy", "```", "",
             "Each step runs the per-token quantisation and the GEMM for every M: about 100 ms of untimed "
             "steps while the clocks settle, the warm-up step, two timed steps and two more with events "
             "around each launch; the small-M GEMMs (M = 1, 16) are also launched 30 times back to back "
             "per M for their per-launch time.  Durations are per dispatch, from the kernel trace; the "
             "median per grid leaves out the first steps, which run before the clocks have risen.", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{_short(r['Name'])[:100]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.2f} |")
    per_grid = {}
    for r in _read_csv(trace_dir, "kernel_trace.csv"):
        k = _short(r["Kernel_Name"])
        if not k.startswith("w4::w4_gemm"):
            continue
        key = (k, int(float(r.get("Grid_Size_X", r.get("Grid_Size", 0)) or 0)))
        per_grid.setdefault(key, []).append(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]))))
    lines += ["", "GEMM launches by grid (threads; one grid per M except M = 1 and 16, which share one); "
              "the last column lists the last eight launches in launch order:", "",
              "| kernel | grid | calls | avg us | median us | last launches us |", "|---|---|---|---|---|---|"]
    for (k, g), v in sorted(per_grid.items(), key=lambda kv: kv[0][1]):
        d = [(e - b) / 1e3 for b, e in sorted(v)]
        med = sorted(d)[len(d) // 2]
        shown = ("..., " if len(d) > 8 else "") + ", ".join(f"{x:.1f}" for x in d[-8:])
        lines.append(f"| `{k[:100]}` | {g} | {len(d)} | {sum(d) / len(d):.1f} | {med:.1f} | {shown} |")
    with open(STATS_MD, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(STATS_MD)


def traffic_for(label: str, Ms) -> "float | None":
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None if there is none or the GEMM sources changed since."""
    try:
        with open(TRAFFIC_MD) as fh:
            text = fh.read()
        data = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None
    if data.get("source_sha256") != sources_sha256():
        return None
    grids = {M: grid_of(label, M) for M in Ms}
    vals = [v["hbm_bytes_per_launch"] for k, v in data["kernels"].items()
            if v.get("hbm_bytes_per_launch") and kernel_matches(k, label)
            and ("skinny" in label or any(k.endswith(f"grid={g}") for g in grids.values()))]
    return round(sum(vals) / len(vals)) if vals else None


def grid_of(label: str, M: int) -> int:
    """Total threads of the GEMM launch for M (the trace's Grid_Size)."""
    m = re.search(r"(\d+)x(\d+) tile", label)
    if not m:
        return -1
    tm, tn = int(m.group(1)), int(m.group(2))
    return ((M + tm - 1) // tm) * ((N + tn - 1) // tn) * 256


def kernel_matches(key: str, label: str) -> bool:
    if "tiled" in label:
        m = re.search(r"(\d+)x(\d+) tile", label)
        mt = int(m.group(1)) // 16 if m else 0
        return "w4_gemm_tiled" in key and f", 4, {mt}, " in key and key.rstrip().endswith(
            "grid=" + key.rsplit("grid=", 1)[1])
    return "w4_gemm_skinny" in key


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed steps for at least this long before the warm-up steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ms", default=",".join(str(m) for m in MS))
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (read + write) to scale HBM counters")
    ap.add_argument("--summarize", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the HBM-traffic summary from rocprofv3 outputs and exit")
    args = ap.parse_args(argv)
    if args.summarize:
        return summarize(*args.summarize)
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library runs on a single MI355X and has no "
              f"multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2
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

    calib = None
    if args.calibrate_copy:
        src = torch.zeros(CALIB_BYTES // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        ce = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        torch.bitwise_not(src, out=dst)                  # warm-up
        ce[0].record()
        torch.bitwise_not(src, out=dst)                  # plain copy kernel: reads and writes 256 MiB
        ce[1].record()
        torch.cuda.synchronize()
        us = ce[0].elapsed_time(ce[1]) * 1e3
        calib = {"bytes_read": CALIB_BYTES, "bytes_written": CALIB_BYTES, "us": round(us, 2),
                 "GBps_read_plus_write": round(2 * CALIB_BYTES / (us * 1e-6) / 1e9, 1)}
        del src, dst

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

    # ---- per-launch durations of the small-M kernel ----------------------
    # A launch of ~20 us bracketed by two events also counts the event-to-
    # kernel dispatch latency (a few us), so the small-M GEMMs are timed again
    # alone: REPS launches back to back (rotating the weight copies) between
    # two events on the launch stream.  Longer kernels keep their in-step
    # figure, where that latency is negligible.
    REPS = 30
    iso_us = {}
    for i, M in enumerate(Ms):
        if plans[M][0] != 1:
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
        path, split, tm, tn = plans[M]
        k_us = iso_us.get(M, g_us)
        per_m.append({"M": M, "kernel": kernel_label(path, split, tm, tn), "k_split": split,
                      "gemm_us_in_step": round(g_us, 2), "quant_us_in_step": round(q_us, 2),
                      "gemm_us": round(k_us, 2), "gemm_timing": "back-to-back" if M in iso_us else "in-step",
                      "gemm_tops": round(ops / (k_us * 1e-6) / 1e12, 2),
                      "weight_GBps": round((N * K / 2) / (k_us * 1e-6) / 1e9, 1),
                      "alg_GBps": round(gemm_alg_bytes(M) / (k_us * 1e-6) / 1e9, 1),
                      "hbm_frac": round(gemm_alg_bytes(M) / (k_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                      "mfma_frac": round(ops / (k_us * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4)})
    value = total_ops / (ms_per_step * 1e-3) / 1e12

    # dominant kernel: the kernel (template instance) with the most time in a step
    by_kernel = {}
    for pm in per_m:
        by_kernel.setdefault(pm["kernel"], []).append(pm)
    dom_name, dom = max(by_kernel.items(), key=lambda kv: sum(pm["gemm_us"] for pm in kv[1]))
    flops = sum(2.0 * pm["M"] * N * K for pm in dom) / len(dom)
    dur = sum(pm["gemm_us"] for pm in dom) / len(dom)
    ach = flops / (dur * 1e-6) / 1e12
    roofline = {"bound": "mfma", "achieved": round(ach, 2), "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
                "frac": round(ach / INT8_PEAK_TOPS, 4), "traffic": traffic_for(dom_name, [pm["M"] for pm in dom]),
                "kernel": dom_name, "launches": [pm["M"] for pm in dom], "avg_launch_us": round(dur, 2),
                "note": "int8 ops (2 per multiply-add) per second; avg_launch_us from a second pass of "
                        "the timed steps with events around each launch on the launch stream"}
    small = [pm for pm in per_m if pm["kernel"].startswith("w4_gemm_skinny")]
    roofline_small = None
    if small:
        b = sum(gemm_alg_bytes(pm["M"]) for pm in small) / len(small)
        dur = sum(pm["gemm_us"] for pm in small) / len(small)
        gb = b / (dur * 1e-6) / 1e9
        roofline_small = {"bound": "hbm", "achieved": round(gb, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                          "frac": round(gb / HBM_PEAK_GBPS, 4),
                          "traffic": traffic_for(small[0]["kernel"], [pm["M"] for pm in small]),
                          "kernel": small[0]["kernel"], "launches": [pm["M"] for pm in small],
                          "avg_launch_us": round(dur, 2),
                          "note": f"avg_launch_us from {REPS} back-to-back launches per M between two events"}

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
