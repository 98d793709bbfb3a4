#!/usr/bin/env python3
"""Measure the tuning table of the FP32 GEMM library on the GPU at hand.

The library's automatic choice for 16-byte-aligned operands looks up a table
from shape classes of (M, N, K) to an MFMA tile configuration, a tile-row
grouping of the work-group order and a split of K over work-groups.  This
script measures that table: for every class it times the candidate plans on a
product of the class's upper bound in each extent, through the library's
``sgemm_f32_ex_config`` entry point, and keeps the fastest.  It is the
autotuning step that "How a Matmul Kernel Gets Fast" describes in its section
"Kernel 9: autotuning" (sweep the tiling parameters, keep the best per
problem), applied to the configurations this library compiles.

Each plan is timed as the benchmark times a step: single launches, each
between its own pair of events, median of at least 11; the candidates of a
class are timed in three interleaved passes and compared by the median of
those.  A candidate replaces
the default plan of its class only when it is faster by more than
``--min-gain`` (5 % by default), so run-to-run noise does not move the table.
Every adopted plan's result is compared against the default plan's result on
the same inputs (same values up to summation order).

Writes ``fp32_sgemm_amd/tuning_table.json`` (the measurements) and
``fp32_sgemm_amd/csrc/sgemm_tuning_table.inc`` (the table compiled into the
library); rebuild the library afterwards.  Usage:

    python fp32_sgemm_amd/tune.py [--classes 0-7] [--min-gain 0.05] [--dry-run]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

CLASS_BOUNDS = [64, 128, 256, 512, 1024, 2048, 4096, 8192]
SPLITS = [1, 2, 4, 8]
GROUPS = [4, 8, 16]
TABLE_JSON = os.path.join(HERE, "tuning_table.json")
TABLE_INC = os.path.join(HERE, "csrc", "sgemm_tuning_table.inc")


def default_plan(M, N):
    """The library's choice without a table: 128x128 tiles unless they give
    fewer than 256 tiles, then 64x64 with two slices in flight; group 8; no
    split."""
    tiles = -(-M // 128) * -(-N // 128)
    return (0 if tiles >= 256 else 4, 8, 1)


NUM_CONFIGS = 7
TILE_BM = {0: 128, 1: 64, 2: 128, 3: 64, 4: 64, 5: 128, 6: 64}
TILE_BN = {0: 128, 1: 64, 2: 64, 3: 128, 4: 64, 5: 128, 6: 64}


def runs_as(plan, M, N, K):
    """The configuration the library runs for a table plan: without a split,
    configuration 0, and configuration 4 on a whole 64x64 grid of at most 1024
    tiles, go to the kernel that loads the operands
    straight into LDS (configurations 8 and 9).  The sweep times what will run
    and stores the table's configuration."""
    cfg, gm, s = plan
    if s == 1:
        if cfg == 0:
            return (8, gm, 1)
        if cfg == 4 and M % 64 == 0 and N % 64 == 0 and (M // 64) * (N // 64) <= 1024:
            return (9, gm, 1)
    return plan


def tiles_of(config, M, N):
    return -(-M // TILE_BM[config]) * -(-N // TILE_BN[config])


def effective_splits(K, s):
    per = -(-K // s)
    per = max(32, -(-per // 32) * 32)
    return -(-K // per)


def candidates(M, N, K):
    out = []
    for cfg in range(NUM_CONFIGS):
        tiles = tiles_of(cfg, M, N)
        for s in SPLITS:
            if cfg == 5 and s > 1:
                continue     # the persistent configuration takes no split
            if s > 1:
                es = effective_splits(K, s)
                # Split only where the grid is short of work-groups and each
                # split keeps at least 128 of K.
                if es != s or K // s < 128 or tiles * s > 4096 or tiles >= 1024:
                    continue
                if s * M * N * 4 > (1 << 30):
                    continue
            out.append((cfg, 8, s))
    return out


class Timer:
    def __init__(self, sg, torch, bufs, stream):
        self.sg, self.torch, self.bufs, self.stream = sg, torch, bufs, stream

    def call(self, plan, M, N, K, C=None):
        cfg, gm, s = runs_as(plan, M, N, K)
        A, B, Cb = self.bufs
        C = Cb if C is None else C
        st = self.sg.sgemm_f32_ex_config(cfg, gm, s, 0, 0, M, N, K, 1.0, A.data_ptr(), K, B.data_ptr(), N,
                                         0.0, C.data_ptr(), N, self.stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"sgemm_f32_ex_config{plan} on {M}x{N}x{K} returned {st}")

    def time(self, plan, M, N, K, budget_ms=4.0):
        """Median duration of single launches, each between its own pair of
        events (the way the benchmark times a step), in microseconds."""
        torch = self.torch
        ev = lambda: torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(self.stream):
            self.call(plan, M, N, K)
            e0, e1 = ev(), ev()
            e0.record(self.stream)
            self.call(plan, M, N, K)
            e1.record(self.stream)
        e1.synchronize()
        one = max(e0.elapsed_time(e1), 1e-3)
        reps = int(min(100, max(11, budget_ms / one)))
        pairs = [(ev(), ev()) for _ in range(reps)]
        with torch.cuda.stream(self.stream):
            for a, b in pairs:
                a.record(self.stream)
                self.call(plan, M, N, K)
                b.record(self.stream)
        pairs[-1][1].synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in pairs)
        return ms[len(ms) // 2] * 1e3


def measure(timer, plans, M, N, K, rounds):
    """Median time of each plan over `rounds` passes that each time every plan
    once, so that a drift of the GPU's state during the sweep does not favour
    the plans timed first."""
    import statistics
    samples = {p: [] for p in plans}
    for _ in range(rounds):
        for p in plans:
            samples[p].append(timer.time(p, M, N, K))
    return {p: statistics.median(v) for p, v in samples.items()}


def dump_table(out):
    """JSON with one line per entry."""
    head = {k: v for k, v in out.items() if k != "entries"}
    lines = ["{"]
    for k, v in head.items():
        lines.append(f" {json.dumps(k)}: {json.dumps(v)},")
    lines.append(' "entries": [')
    ents = [json.dumps(e) for e in out["entries"]]
    lines.append(",\n".join("  " + e for e in ents))
    lines.append(" ]")
    lines.append("}")
    return "\n".join(lines) + "\n"


def write_inc(entries, path):
    # A class whose measured winner is the default plan keeps the default
    # choice, which depends on the actual extents (the tile count), rather
    # than the plan that was default at the class bound.
    grid = {}
    for e in entries:
        plan = [e["config"], e["group_m"], e["splits"]]
        if plan != list(e["default"]):
            grid[(e["mc"], e["nc"], e["kc"])] = tuple(plan)
    n = len(CLASS_BOUNDS)
    lines = [
        "// Tuning table measured by fp32_sgemm_amd/tune.py (see tuning_table.json for the",
        "// timings).  Index [m][n][k] by shape class; entry {config, group_m, splits};",
        "// {-1, -1, -1} means the default choice (the class's measured winner was the default).",
        "constexpr bool kHaveTunedTable = true;",
        "constexpr TunedEntry kTunedTable[kNumClasses][kNumClasses][kNumClasses] = {",
    ]
    for mc in range(n):
        lines.append("    {")
        for nc in range(n):
            row = []
            for kc in range(n):
                c, g, s = grid.get((mc, nc, kc), (-1, -1, -1))
                row.append(f"{{{c}, {g}, {s}}}")
            lines.append("        {" + ", ".join(row) + "},")
        lines.append("    },")
    lines.append("};")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser(description="measure the tuning table")
    ap.add_argument("--classes", default="0-7", help="range of classes per extent, e.g. 3-6")
    ap.add_argument("--min-gain", type=float, default=0.05)
    ap.add_argument("--rounds", type=int, default=3, help="interleaved timing passes per class")
    ap.add_argument("--dry-run", action="store_true", help="measure and print, write nothing")
    ap.add_argument("--out-dir", default=None,
                    help="write tuning_table.json and sgemm_tuning_table.inc here instead of "
                         "into the package")
    args = ap.parse_args()
    lo, hi = (int(v) for v in args.classes.split("-"))

    import torch

    import fp32_sgemm_amd as sg

    if not torch.cuda.is_available():
        sys.exit("tune.py needs a GPU")
    dev = torch.device("cuda:0")
    big = CLASS_BOUNDS[hi]
    g = torch.Generator(device="cpu").manual_seed(1234)
    A = (torch.rand(big * big, generator=g) * 2 - 1).to(dev)
    B = (torch.rand(big * big, generator=g) * 2 - 1).to(dev)
    C = torch.empty(big * big, device=dev)
    C2 = torch.empty(big * big, device=dev)
    stream = torch.cuda.Stream(dev)
    timer = Timer(sg, torch, (A, B, C), stream)

    entries = []
    t_start = time.time()
    for mc in range(lo, hi + 1):
        for nc in range(lo, hi + 1):
            for kc in range(lo, hi + 1):
                M, N, K = CLASS_BOUNDS[mc], CLASS_BOUNDS[nc], CLASS_BOUNDS[kc]
                d = default_plan(M, N)
                plans = [d] + [c for c in candidates(M, N, K) if c != d]
                results = measure(timer, plans, M, N, K, args.rounds)
                best = min(results, key=results.get)
                if tiles_of(best[0], M, N) * best[2] >= 256:
                    extra = [(best[0], gm, best[2]) for gm in GROUPS if (best[0], gm, best[2]) not in results]
                    if extra:
                        results.update(measure(timer, [d, best] + extra, M, N, K, args.rounds))
                    best = min(results, key=results.get)
                t_def = results[d]
                if results[best] > t_def * (1 - args.min_gain):
                    best = d
                # The adopted plan must give the default plan's values (up to
                # summation order).
                if best != d:
                    timer.call(d, M, N, K)
                    timer.call(best, M, N, K, C=C2)
                    torch.cuda.synchronize()
                    x, y = C[:M * N], C2[:M * N]
                    rel = float((x - y).abs().max() / (x.abs().max() + 1e-30))
                    if rel > 1e-5:
                        raise RuntimeError(f"plan {best} disagrees with {d} on {M}x{N}x{K}: {rel}")
                e = {"mc": mc, "nc": nc, "kc": kc, "shape": [M, N, K], "config": best[0],
                     "group_m": best[1], "splits": best[2], "us": round(results[best], 2),
                     "default": list(d), "default_us": round(t_def, 2),
                     "tflops": round(2 * M * N * K / results[best] / 1e6, 2),
                     "tried": len(results)}
                entries.append(e)
                print(json.dumps(e), flush=True)
    dt = time.time() - t_start
    props = torch.cuda.get_device_properties(dev)
    out = {"device": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
           "class_bounds": CLASS_BOUNDS, "min_gain": args.min_gain, "seconds": round(dt, 1),
           "library_version": sg.sgemm_f32_version(), "entries": entries}
    if args.dry_run:
        return
    tj, ti = TABLE_JSON, TABLE_INC
    if args.out_dir:
        os.makedirs(args.out_dir, exist_ok=True)
        tj = os.path.join(args.out_dir, os.path.basename(TABLE_JSON))
        ti = os.path.join(args.out_dir, os.path.basename(TABLE_INC))
    with open(tj, "w") as f:
        f.write(dump_table(out))
    write_inc(entries, ti)
    print(f"wrote {tj} and {ti} ({len(entries)} classes, {dt:.0f} s); rebuild the library",
          flush=True)


if __name__ == "__main__":
    main()
