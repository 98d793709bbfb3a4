#!/usr/bin/env python3
"""Benchmark: FP32 SGEMM throughput on one MI355X.

One step is one call of the library's C entry point ``sgemm_f32`` on the
4096 x 4096 x 4096 workload (A, B, C standard normal, C = 1.5*A*B - 0.5*C, in
place), with all inputs resident in device memory.  Prints one JSON line.
``--operands nt|tn|tt`` stores A and/or B transposed and times ``sgemm_f32_ex``
on the same product.

Timing: W untimed warm-up steps, then K timed steps bracketed by device
synchronisation; each launch is also bracketed by HIP events recorded on the
stream the kernel runs on, which give the kernel's average duration for the
roofline figure.  The FLOP count is 2*M*N*K per step (the scaling by alpha and
beta is not counted, "How a Matmul Kernel Gets Fast", section 1 and "Writing a
Fast Matmul in CUDA, Step by Step", section "Step 1").

The CPU baseline is the float64 oracle timed on the host's cores on a bounded
sample of the same product (its first rows), reported beside the GPU number.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FP32 SGEMM TFLOP/s at 4096^3 on 1 MI355X; % of FP32 peak"
PEAK_FP32_TFLOPS = 157.3          # MI355X dense FP32 (vector and matrix), datasheet
PEAK_16BIT_TFLOPS = 2500.0        # MI355X dense BF16 / FP16 matrix, datasheet
METRIC_16 = "GEMM TFLOP/s with {} inputs and FP32 accumulation at {} on 1 MI355X"
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ("fp32_sgemm_amd/csrc/sgemm_mfma.hip", "fp32_sgemm_amd/csrc/gemm_internal.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_mfma_large_square4096_ab.txt")


# --- closed-form work and byte counts ------------------------------------------------
def gemm_flops(M: int, N: int, K: int) -> int:
    """Multiply-adds counted as 2 FLOP each: 2*M*N*K."""
    return 2 * M * N * K


def gemm_min_bytes(M: int, N: int, K: int, reads_c: bool, elem: int = 4) -> int:
    """Bytes that must cross HBM at least once: read A and B, write C, and read
    C too when beta != 0 ("How a Matmul Kernel Gets Fast", section 2)."""
    return elem * (M * K + K * N + M * N * (2 if reads_c else 1))


def arithmetic_intensity(M: int, N: int, K: int, reads_c: bool) -> float:
    return gemm_flops(M, N, K) / gemm_min_bytes(M, N, K, reads_c)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when that summary is missing or was taken on other kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


# --- CPU baseline (the oracle on a bounded sample) -----------------------------------
def cpu_baseline(A, B, C0, alpha, beta, target_s: float):
    import oracle

    M, K = A.shape
    N = B.shape[1]
    cores = oracle.num_threads()
    rows = min(M, max(cores, 8))
    t0 = time.perf_counter()
    oracle.sgemm_ref(A[:rows], B, alpha, beta, None if C0 is None else C0[:rows])
    dt = time.perf_counter() - t0
    per_row = dt / rows
    R = int(min(M, max(rows, target_s / max(per_row, 1e-9))))
    R = max(cores, (R // cores) * cores) if R >= cores else R
    R = min(R, M)
    t0 = time.perf_counter()
    oracle.sgemm_ref(A[:R], B, alpha, beta, None if C0 is None else C0[:R])
    dt = time.perf_counter() - t0
    return {
        "value": round(gemm_flops(R, N, K) / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"rows 0..{R - 1} of the {M}x{N}x{K} product ({R * N} outputs, "
                  f"float64 accumulation, {dt:.1f} s)",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, help="workload name (default: the 4096^3 headline)")
    ap.add_argument("--shape", default=None, metavar="MxNxK",
                    help="time another shape instead (uniform[-1,1) inputs, alpha 1, beta 0)")
    ap.add_argument("--variant", default="auto",
                    help="auto | mfma_large | mfma_small | valu | skinny | mfma_scalar")
    ap.add_argument("--operands", default="nn", choices=["nn", "nt", "tn", "tt"],
                    help="operand forms: t = stored transposed (A as K x M, B as N x K), "
                         "timed through sgemm_f32_ex")
    ap.add_argument("--inputs16", default=None, choices=["bf16", "f16"],
                    help="time gemm16_f32 instead: A and B stored in this 16-bit format, "
                         "FP32 accumulation and C")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time for the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate", type=int, default=1, metavar="COPIES",
                    help="cycle the steps over this many copies of B (with 5 or more, the "
                         "copies exceed the 256 MB Infinity Cache for the skinny workload)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the GEMM, run 10 plain device copies of MIB MiB "
                         "(x*1 elementwise) to calibrate HBM byte counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp32_sgemm_amd as sg
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration * 1024 * 1024 // 4
        src = torch.randn(n, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(10):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n,
                          "launches": 10}), flush=True)
        return
    names = {sg.sgemm_f32_variant_name(i): i for i in range(sg.NUM_VARIANTS)}
    if args.variant not in names:
        sys.exit(f"unknown variant {args.variant}")
    variant = names[args.variant]

    if args.shape:
        M, N, K = (int(v) for v in args.shape.lower().split("x"))
        w = workloads.custom(M, N, K, dist="uniform", seed=99, name=f"shape{M}x{N}x{K}")
    else:
        w = workloads.WORKLOADS[args.workload or workloads.HEADLINE]
    A, B, C0 = workloads.make_inputs(w)
    ta, tb = int(args.operands[0] == "t"), int(args.operands[1] == "t")
    kind16 = {"bf16": 1, "f16": 2}.get(args.inputs16)
    if kind16:
        A, B = workloads.to_16bit(A, kind16), workloads.to_16bit(B, kind16)
    As = np.ascontiguousarray(A.T) if ta else A
    Bs = np.ascontiguousarray(B.T) if tb else B
    dev = torch.device("cuda:0")
    to_dev = (lambda x: torch.from_numpy(x.view(np.int16)).to(dev)) if kind16 else (lambda x: torch.from_numpy(x).to(dev))
    dA = to_dev(As)
    dBs = [to_dev(Bs) for _ in range(max(1, args.rotate))]
    dB = dBs[0]
    dC = torch.from_numpy(C0).to(dev) if C0 is not None else torch.empty(w.M, w.N, device=dev)
    lda, ldb, ldc = As.shape[1], Bs.shape[1], w.N
    stream = torch.cuda.Stream(dev)
    s_handle = stream.cuda_stream
    chosen = variant if variant else sg.sgemm_f32_ex_select(ta, tb, w.M, w.N, w.K, w.alpha, dA.data_ptr(),
                                                            lda, dB.data_ptr(), ldb)

    plan = None
    if variant in (0, sg.MFMA_TUNED):
        st, pv, pc, pg, ps = sg.sgemm_f32_ex_plan(ta, tb, w.M, w.N, w.K, w.alpha, dA.data_ptr(), lda,
                                                  dB.data_ptr(), ldb)
        if st == 0 and pv not in (0, sg.SKINNY, sg.VALU):
            plan = {"config": sg.sgemm_f32_config_name(pc), "group_m": pg, "splits": ps}
    counter = [0]

    def step():
        b = dBs[counter[0] % len(dBs)]
        counter[0] += 1
        if kind16:
            st = sg.gemm16_f32(kind16, ta, tb, w.M, w.N, w.K, w.alpha, dA.data_ptr(), lda, b.data_ptr(), ldb,
                               w.beta, dC.data_ptr(), ldc, s_handle)
        elif ta or tb:
            st = sg.sgemm_f32_ex_variant(variant, ta, tb, w.M, w.N, w.K, w.alpha, dA.data_ptr(), lda,
                                         b.data_ptr(), ldb, w.beta, dC.data_ptr(), ldc, s_handle)
        else:
            st = sg.sgemm_f32_variant(variant, w.M, w.N, w.K, w.alpha, dA.data_ptr(), lda,
                                      b.data_ptr(), ldb, w.beta, dC.data_ptr(), ldc, s_handle)
        if st != 0:
            raise RuntimeError(f"sgemm_f32 returned {st}")

    torch.cuda.synchronize(dev)
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize(dev)

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            starts[i].record(stream)
            step()
            ends[i].record(stream)
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()

    elapsed = t1 - t0
    flops = gemm_flops(w.M, w.N, w.K)
    value = flops * args.steps / elapsed / 1e12
    kern_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    kern_avg_s = float(np.mean(kern_ms)) / 1e3
    achieved = flops / kern_avg_s / 1e12

    peak = PEAK_16BIT_TFLOPS if kind16 else PEAK_FP32_TFLOPS
    memory_bound = arithmetic_intensity(w.M, w.N, w.K, w.beta != 0) < peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if kind16 and not memory_bound:
        roofline = {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4)}
    elif memory_bound:
        ach_gbs = gemm_min_bytes(w.M, w.N, w.K, w.beta != 0) / kern_avg_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(ach_gbs, 2), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(ach_gbs / PEAK_HBM_GBS, 4)}
    else:
        # The VALU comparison kernel is bound by the vector FP32 rate; every
        # other kernel by the FP32 matrix-core rate (the same datasheet number).
        bound = "alu" if chosen == sg.VALU else "mfma"
        roofline = {"bound": bound, "achieved": round(achieved, 3), "peak": PEAK_FP32_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_TFLOPS, 4)}
    headline_kernel = w.name == workloads.HEADLINE and chosen == 1 and not (ta or tb) and not kind16
    roofline["traffic"] = measured_traffic() if headline_kernel else None
    roofline["kernel_avg_ms"] = round(kern_avg_s * 1e3, 5)

    if kind16:
        chosen_name = "gemm16_" + args.inputs16
        plan = None
    else:
        chosen_name = sg.sgemm_f32_variant_name(chosen)
    out = {
        "metric": METRIC_16.format(args.inputs16, f"{w.M}x{w.N}x{w.K}") if kind16 else METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.inputs16 + " in, f32 accumulate" if kind16 else "f32",
        "data": "synthetic",
        "pct_of_fp32_peak": None if kind16 else round(100 * value / PEAK_FP32_TFLOPS, 2),
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "alpha": w.alpha,
                   "beta": w.beta, "inputs": w.dist, "operands": args.operands,
                   "variant": chosen_name, "plan": plan,
                   "b_copies": len(dBs), "parallelism": "single GPU"},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline and not kind16:
        out["cpu_baseline"] = cpu_baseline(A, B, C0, w.alpha, w.beta, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
