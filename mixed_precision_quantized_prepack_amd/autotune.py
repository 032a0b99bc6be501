"""Schedule autotuning: measure the kernel schedules of each (shape, M bucket)
on the GPU and write the built-in schedule table.

A schedule is (path, K split, tile rows, strips per wave), the fields of the
library's tuning options (path 3, the streaming kernel, reads the strips
field as 16-column blocks per wave).  For every M bucket the module times the
heuristic's choice and each schedule that fits the problem, at the bucket's
largest M, and keeps an entry only where the best schedule beats the
heuristic by a margin (the heuristic stays in charge elsewhere).

    python -m mixed_precision_quantized_prepack_amd.autotune --out results.json   # on a GPU
    python -m mixed_precision_quantized_prepack_amd.autotune --write-table results.json

The second form writes ``csrc/w4_schedule_table.inc``; rebuild the library
afterwards.  Inputs are random: timings do not depend on the values.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import mixed_precision_quantized_prepack_amd as w4

TABLE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "w4_schedule_table.inc")

# (name, activation dtype code, group size (-1 = per channel), N, K, scale dtype, out dtype)
SHAPES = [
    ("w4a8_i8_pc_8192x21760", w4.I8, -1, 8192, 21760, "f32", "f16"),
    ("w4a8_i8_g128_qkv_12288x4096", w4.I8, 128, 12288, 4096, "f16", "f16"),
    ("w4a8_i8_g128_o_4096x4096", w4.I8, 128, 4096, 4096, "f16", "f16"),
    ("w4a8_i8_g128_gateup_22016x4096", w4.I8, 128, 22016, 4096, "f16", "f16"),
    ("w4a8_i8_g128_down_4096x11008", w4.I8, 128, 4096, 11008, "f16", "f16"),
    ("w4a8_fp8_g128_28672x8192", w4.FP8_E4M3, 128, 28672, 8192, "f32", "bf16"),
    ("w4a16_bf16_g128_4096x4096", w4.BF16, 128, 4096, 4096, "bf16", "bf16"),
    ("w4a16_f16_pc_8192x8192", w4.F16, -1, 8192, 8192, "f16", "f16"),
]

BUCKETS = [(1, 1), (2, 4), (5, 8), (9, 16), (17, 32), (33, 64), (65, 128), (129, 256), (257, 512),
           (513, 1024), (1025, 2048), (2049, 4096), (4097, 8192)]

DTYPE_NAMES = {w4.I8: "W4_I8", w4.FP8_E4M3: "W4_FP8_E4M3", w4.F16: "W4_F16", w4.BF16: "W4_BF16"}
OPTION_KEYS = ("force_path", "splitk", "tiled_bm", "skinny_strips")


def _set_schedule(path=0, splitk=0, tile_m=0, strips=0):
    for k, v in zip(OPTION_KEYS, (path, splitk, tile_m, strips)):
        w4.set_option(k, v)


def candidates(a_dtype: int, grouped: bool, M: int, N: int, K: int):
    """Schedules (path, splitk, tile_m, strips) that fit the problem."""
    byte = a_dtype in (w4.I8, w4.FP8_E4M3)
    out = []
    if M <= 16:
        smax = 16 if (byte and not grouped) else 8
        for strips in (1, 2):
            for s in (1, 2, 4, 8, 16):
                if s <= smax and s <= K // 128:
                    out.append((1, s, 0, strips))
    # tiled: the default tile for the rows (0), or 128 columns (2 blocks per
    # wave) for 8-bit operands with 64-row tiles
    for tm, nt in (((64, 0), (64, 2), (128, 0)) if byte else ((64, 0),)):
        for s in (1, 2, 4, 8, 16):
            if s <= K // 128:
                out.append((2, s, tm, nt))
    # the ping-pong kernel (int8 per channel; other problems refuse it)
    if a_dtype == w4.I8 and not grouped and M > 64:
        for tm in (128, 256):
            for s in (1, 2, 4, 8):
                if s <= K // 128:
                    out.append((4, s, tm, 0))
    if byte and 16 < M <= 256:
        for tm in (32, 64, 128):
            for nt in ((2,) if tm == 128 else (2, 4)):
                for s in (0, 1, 2, 4, 8, 16):
                    if s <= K // 128:
                        out.append((3, s, tm, nt))
    fits = []
    gs = 128 if grouped else -1
    for c in out:
        _set_schedule(*c)
        try:
            w4.gemm_plan(M, N, K, gs, a_dtype)
            fits.append(c)
        except w4.W4Error:
            pass
    _set_schedule()
    return fits


class Problem:
    """Device buffers for one shape at its largest M, with enough weight
    copies that consecutive launches read the weights from HBM."""

    def __init__(self, a_dtype, gs, N, K, s_dtype, out_dtype, m_max, torch):
        self.t = torch
        dev = torch.device("cuda")
        self.a_dtype, self.gs, self.N, self.K = a_dtype, gs, N, K
        G = 1 if gs == -1 else K // gs
        td = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
        wbytes = N * K // 2
        self.copies = max(2, min(64, math.ceil((1 << 30) / wbytes)))
        self.packed = [torch.randint(0, 256, (wbytes,), dtype=torch.uint8, device=dev)
                       for _ in range(self.copies)]
        shape = (N,) if gs == -1 else (N, G)
        self.scales = (torch.rand(shape, device=dev) * 0.015 + 0.005).to(td[s_dtype])
        self.out = torch.empty((m_max, N), dtype=td[out_dtype], device=dev)
        if a_dtype == w4.I8:
            self.a = torch.randint(-127, 128, (m_max, K), dtype=torch.int8, device=dev)
            self.sa = torch.rand((m_max,), device=dev) * 0.01 + 0.001
        elif a_dtype == w4.FP8_E4M3:
            self.a = (torch.randn((m_max, K), device=dev) * 64).to(torch.float8_e4m3fn).view(torch.uint8)
            self.sa = torch.rand((m_max,), device=dev) * 0.01 + 0.001
        else:
            self.a = torch.randn((m_max, K), device=dev).to(td["f16" if a_dtype == w4.F16 else "bf16"])
            self.zeros = torch.randint(0, 16, (N, G), device=dev).to(self.a.dtype)
            self.scales = self.scales.to(self.a.dtype)
        self.ws = None

    def launcher(self, M: int):
        t = self.t
        need = w4.gemm_workspace_bytes(M, self.N, self.K, self.gs, self.a_dtype)
        if need and (self.ws is None or self.ws.numel() < need):
            self.ws = t.empty(need, dtype=t.uint8, device="cuda")
        ws = self.ws if need else None
        a, out = self.a[:M], self.out[:M]
        if self.a_dtype in (w4.I8, w4.FP8_E4M3):
            sa = self.sa[:M]
            return lambda i: w4.w4a8_gemm(a, sa, self.packed[i % self.copies], self.scales, self.gs, out.dtype,
                                          out=out, workspace=ws)
        return lambda i: w4.w4a16_gemm(a, self.packed[i % self.copies], self.scales, self.zeros, self.gs,
                                       out=out, workspace=ws)


def _time_us(torch, fn, reps: int) -> float:
    """Average launch time of `reps` launches captured in a HIP graph (so
    the host's launch rate does not bound short kernels), fastest of two
    replays."""
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
    best = float("inf")
    for _ in range(2):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e3 / reps)
    del g
    return best


def tune(shapes, buckets, trials: int, margin: float, log=print):
    import torch
    results = []
    for name, a_dtype, gs, N, K, s_dtype, out_dtype in shapes:
        grouped = gs != -1
        m_top = max(hi for _, hi in buckets)
        prob = Problem(a_dtype, gs, N, K, s_dtype, out_dtype, m_top, torch)
        # raise the clocks before the first measurement
        w4.set_option("schedule_table", 0)
        _set_schedule()
        fn = prob.launcher(16)
        t_end = time.time() + 0.2
        while time.time() < t_end:
            _time_us(torch, fn, 20)
        for lo, hi in buckets:
            M = hi
            cands = candidates(a_dtype, grouped, M, N, K)
            heur = w4.gemm_plan(M, N, K, gs, a_dtype)
            best = {}
            # the heuristic is entry None; trials alternate between candidates
            order = [None] + cands
            est = None
            for _ in range(trials):
                for c in order:
                    _set_schedule(*(c or (0, 0, 0, 0)))
                    fn = prob.launcher(M)
                    if est is None:
                        est = _time_us(torch, fn, 3)
                    reps = max(5, min(100, int(3000.0 / max(est, 1.0))))
                    us = _time_us(torch, fn, reps)
                    best[c] = min(best.get(c, float("inf")), us)
            _set_schedule()
            h_us = best.pop(None)
            c_best = min(best, key=best.get) if best else None
            b_us = best[c_best] if c_best else h_us
            keep = c_best is not None and b_us < h_us * (1.0 - margin) and not same_schedule(heur, c_best)
            row = {"shape": name, "a_dtype": a_dtype, "grouped": grouped, "N": N, "K": K, "m_lo": lo,
                   "m_hi": hi, "M": M, "heuristic": list(heur), "heuristic_us": round(h_us, 2),
                   "best": list(c_best) if c_best else None, "best_us": round(b_us, 2), "keep": keep,
                   "all_us": {",".join(map(str, c)): round(v, 2) for c, v in best.items()}}
            log(f"{name} M={M}: heuristic {heur} {h_us:.2f} us, best {c_best} {b_us:.2f} us"
                f"{'  -> entry' if keep else ''}")
            results.append(row)
        del prob
        torch.cuda.empty_cache()
    w4.set_option("schedule_table", 1)
    return results


def same_schedule(plan, cand) -> bool:
    """Whether a candidate (path, splitk, tile_m, strips) is the plan
    (path, splitk, tile_m, tile_n) itself: then a faster timing is noise."""
    path, split, tm, tn = plan
    cp, cs, ctm, cst = cand
    if cp != path or (cs != split and cs != 0):
        return False
    if path in (2, 4):
        return ctm == tm and (cst * 64 == tn or cst == 0)
    if path == 3:
        return (ctm == tm or ctm == 0) and (cst * 64 == tn or cst == 0)
    return cst * 16 == tn


def write_table(results, path: str = TABLE_PATH, margin: float = None) -> int:
    """Write the entries of a results file; `margin`, when given, re-decides
    which entries to keep from the recorded timings."""
    lines = ["// Schedule table: {a_dtype, grouped, N, K, m_lo, m_hi, path, splitk, tile_m, strips}.",
             "// Written by mixed_precision_quantized_prepack_amd/autotune.py from MI355X measurements;",
             "// each entry beat the heuristic's schedule at m_hi (timings in the comment)."]
    n = 0
    for r in results:
        keep = r["keep"] if margin is None else (r["best"] is not None and
                                                 r["best_us"] < r["heuristic_us"] * (1.0 - margin))
        if not keep or same_schedule(r["heuristic"], r["best"]):
            continue
        p, s, tm, st = r["best"]
        lines.append(f"    {{{DTYPE_NAMES[r['a_dtype']]}, {int(r['grouped'])}, {r['N']}, {r['K']}, {r['m_lo']}, "
                     f"{r['m_hi']}, {p}, {s}, {tm}, {st}}},  // {r['shape']}: {r['best_us']} us vs "
                     f"{r['heuristic_us']} us")
        n += 1
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return n


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--out", help="measure on the GPU and write the results (JSON) here")
    ap.add_argument("--write-table", metavar="RESULTS", help="write the built-in table from a results file")
    ap.add_argument("--shapes", default="", help="comma-separated shape names (default: all)")
    ap.add_argument("--trials", type=int, default=3)
    ap.add_argument("--margin", type=float, default=0.03,
                    help="keep an entry when it is this fraction faster than the heuristic")
    args = ap.parse_args(argv)
    if args.write_table:
        with open(args.write_table) as f:
            n = write_table(json.load(f)["results"], margin=args.margin)
        print(f"wrote {n} entries to {TABLE_PATH}")
        return 0
    if not args.out:
        ap.error("give --out (measure) or --write-table")
    shapes = [s for s in SHAPES if not args.shapes or s[0] in args.shapes.split(",")]
    res = tune(shapes, BUCKETS, args.trials, args.margin, log=lambda s: print(s, flush=True))
    with open(args.out, "w") as f:
        json.dump({"margin": args.margin, "trials": args.trials, "results": res}, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
