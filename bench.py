#!/usr/bin/env python3
"""Benchmark: FP32 SGEMM throughput on one MI355X.

One step is one call of the library's C entry point ``sgemm_f32`` on the
4096 x 4096 x 4096 workload (A, B, C standard normal, C = 1.5*A*B - 0.5*C, in
place), with all inputs resident in device memory.  Prints one JSON line.
``--operands nt|tn|tt`` stores A and/or B transposed and times ``sgemm_f32_ex``
on the same product.

Timing follows the pages' method ("Writing a Fast Matmul in CUDA, Step by
Step", section "Step 1: the problem and the yardstick"): the GPU starts in a
low-power state, so the step is first launched back to back for a fixed time
(``--prewarm-seconds``, 0.6 s by default) before anything is counted.  Then W
untimed warm-up steps and K timed steps bracketed by device synchronisation
give ``value``; one pair of HIP events on the kernel's stream around the K
steps gives the kernel's average duration for the roofline figure.  The pages
bracket every launch with events; on this GPU a timing event between two
kernels costs several microseconds of GPU time, so that statistic (the median
of the last three quarters of the launches) comes from a second pass of K
launches, each between its own events, not counted in the value.
Three further rounds of back-to-back launches (events around each, the median
of each round's last three quarters, then the median over rounds) are run for
this library and, interleaved with it under the same warm state, for the
vendor libraries as context.  The FLOP count is 2*M*N*K per step (the scaling
by alpha and beta is not counted, "How a Matmul Kernel Gets Fast", section 1
and the same page's "Step 1").

Parity in the same run: after the timing, C is reset to its initial contents,
the step runs once more, and every element of C is compared with the float64
oracle (within the error bound, or bit for bit for integer-valued inputs), as
the pages check each kernel against a float64 evaluation.  That oracle run is
also the CPU baseline: the oracle timed on the host's cores on the whole
product, plus one thread on a bounded part of it.

Context (not the product): the same product on the same inputs and stream
through rocBLAS ``sgemm`` and through torch's FP32 ``addmm`` (hipBLASLt), and
the GPU's shader clock read with amd-smi while the kernel runs, which gives the
clock-adjusted FP32 peak (256 CUs x 256 FLOP per clock x clock).
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
# The headline plan's kernel (configuration 7) and the tile mapping it uses.
KERNEL_SOURCES = ("fp32_sgemm_amd/csrc/sgemm_big.hip", "fp32_sgemm_amd/csrc/gemm_internal.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_mfma_big_square4096_ab.txt")


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


def kernel_source_hash(sources=None) -> str:
    """Hash of the kernel sources with // comments and blank lines removed, so
    that editing a comment does not invalidate the recorded counters."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        text = sources[rel] if sources else open(os.path.join(ROOT, rel), encoding="utf-8").read()
        for line in text.splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
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


# --- launch timing -------------------------------------------------------------------
def prewarm(torch, stream, call, seconds: float) -> float:
    """Launches `call` back to back on `stream` until `seconds` of wall time
    (synchronised) have passed; returns the time spent."""
    t0 = time.perf_counter()
    batch = 1
    with torch.cuda.stream(stream):
        while True:
            for _ in range(batch):
                call()
            stream.synchronize()
            dt = time.perf_counter() - t0
            if dt >= seconds:
                return dt
            batch = min(batch * 2, 256)


def event_launches(torch, stream, call, n: int):
    """`n` launches back to back, each between its own pair of events on
    `stream`; returns the per-launch durations in ms, in launch order."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    stream.synchronize()
    with torch.cuda.stream(stream):
        for a, b in evs:
            a.record(stream)
            call()
            b.record(stream)
    stream.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def median_last_three_quarters(ms):
    """The pages' statistic: the median of the launches after the first quarter."""
    tail = sorted(ms[len(ms) // 4:])
    return tail[len(tail) // 2]


def timed_rounds(torch, stream, calls: dict, est_ms: dict, round_s: float, rounds: int = 3,
                 max_launches: int = 2000):
    """Interleaved rounds: in each round every call in `calls` runs back to
    back for about `round_s` seconds (at most `max_launches` launches).
    Returns {name: {"rounds_ms": [median of last 3/4 per round], "all_ms": [...]}}."""
    out = {k: {"rounds_ms": [], "all_ms": []} for k in calls}
    for _ in range(rounds):
        for name, call in calls.items():
            n = int(min(max_launches, max(20, round_s / max(est_ms[name] * 1e-3, 1e-7))))
            ms = event_launches(torch, stream, call, n)
            out[name]["rounds_ms"].append(median_last_three_quarters(ms))
            out[name]["all_ms"].extend(ms)
    return out


# --- vendor libraries on the same GPU (context, not the product) ---------------------
def library_calls16(torch, w, ta, tb, dA, dBs, kind16):
    """torch's matmul of the same 16-bit operand views with an FP32 output
    (hipBLASLt).  It computes the plain product (alpha 1, beta 0: torch's mm
    with an FP32 output of 16-bit inputs takes neither), so it does less work
    than a workload with beta != 0."""
    dt = torch.bfloat16 if kind16 == 1 else torch.float16
    Aop = dA.view(dt).t() if ta else dA.view(dt)
    Bops = [b.view(dt).t() if tb else b.view(dt) for b in dBs]
    out_c = torch.empty(w.M, w.N, device=dA.device)
    turn = [0]

    def tm():
        b = Bops[turn[0] % len(Bops)]
        turn[0] += 1
        torch.mm(Aop, b, out_dtype=torch.float32, out=out_c)
    try:
        tm()
        torch.cuda.synchronize()
    except (RuntimeError, TypeError) as e:
        return {}, {"torch_mm_fp32_out": {"error": str(e)[:200]}}
    return {"torch_mm_fp32_out": tm}, {"torch_mm_fp32_out": {"note": "plain product (alpha 1, beta 0)"}}


def library_calls(torch, w, ta, tb, dA, lda, dBs, ldb, C0, stream):
    """rocBLAS sgemm and torch's FP32 addmm (hipBLASLt) on the same product,
    inputs and stream, as callables, plus notes.  rocBLAS is column-major: the
    row-major product C = op(A) op(B) is the column-major C^T = op(B)^T op(A)^T,
    so B is passed first with its own transpose flag (rocBLAS operation 111 =
    none, 112 = transpose); its operand mapping is checked once against
    torch's product of the same views.  Each library call takes the next of the
    B copies in turn, as the timed steps do."""
    import ctypes

    calls, notes = {}, {}
    dB = dBs[0]
    turn = [0]

    def next_b():
        b = dBs[turn[0] % len(dBs)]
        turn[0] += 1
        return b
    dC = (torch.from_numpy(C0).to(dA.device) if C0 is not None
          else torch.zeros(w.M, w.N, device=dA.device))
    try:
        lib = ctypes.CDLL("librocblas.so")
        handle = ctypes.c_void_p()
        if lib.rocblas_create_handle(ctypes.byref(handle)) != 0:
            raise RuntimeError("rocblas_create_handle failed")
        lib.rocblas_set_stream(handle, ctypes.c_void_p(stream.cuda_stream))
        i, p = ctypes.c_int, ctypes.c_void_p
        lib.rocblas_sgemm.argtypes = [p, i, i, i, i, i, p, p, i, p, i, p, p, i]
        al, be = ctypes.c_float(w.alpha), ctypes.c_float(w.beta)
        op_a, op_b = (112 if ta else 111), (112 if tb else 111)

        def roc():
            st = lib.rocblas_sgemm(handle, op_b, op_a, w.N, w.M, w.K, ctypes.byref(al), next_b().data_ptr(), ldb,
                                   dA.data_ptr(), lda, ctypes.byref(be), dC.data_ptr(), w.N)
            if st != 0:
                raise RuntimeError(f"rocblas_sgemm returned {st}")

        z = ctypes.c_float(0.0)
        with torch.cuda.stream(stream):
            lib.rocblas_sgemm(handle, op_b, op_a, w.N, w.M, w.K, ctypes.byref(al), dB.data_ptr(), ldb,
                              dA.data_ptr(), lda, ctypes.byref(z), dC.data_ptr(), w.N)
            ref = w.alpha * ((dA.t() if ta else dA) @ (dB.t() if tb else dB))
        torch.cuda.synchronize()
        agree = bool(((dC - ref).abs().max() <= 1e-3 * ref.abs().max().clamp_min(1e-30)).item())
        del ref
        calls["rocblas_sgemm"] = roc
        notes["rocblas_sgemm"] = {"same_product": agree}
    except (OSError, AttributeError, RuntimeError) as e:
        notes["rocblas_sgemm"] = {"error": str(e)}
    Aop = dA.t() if ta else dA
    torch.backends.cuda.matmul.allow_tf32 = False

    def tm():
        b = next_b()
        dC.addmm_(Aop, b.t() if tb else b, beta=w.beta, alpha=w.alpha)

    calls["torch_addmm"] = tm
    notes["torch_addmm"] = {}
    return calls, notes


def gfx_clock_mhz(torch, step, stream, kern_s):
    """Shader clock of the GPU while the benchmarked kernel runs back to back:
    a second thread keeps launching it for about 2 s while amd-smi reads the
    current clock of each XCD after 1.2 s and 1.6 s (its figure lags the
    hardware by up to about a second).  Returns (mean MHz over XCDs and
    readings, the readings) or (None, reason)."""
    import shutil
    import subprocess
    import threading

    tool = shutil.which("amd-smi")
    if tool is None:
        return None, "amd-smi not found"
    stop = threading.Event()
    batch = int(min(1000, max(1, 0.01 / max(kern_s, 1e-6))))

    def feeder():
        while not stop.is_set():
            for _ in range(batch):
                step()
            stream.synchronize()

    th = threading.Thread(target=feeder, daemon=True)
    readings, err = [], None
    t_start = time.perf_counter()
    th.start()
    try:
        for at in (1.2, 1.6):
            time.sleep(max(0.0, at - (time.perf_counter() - t_start)))
            p = subprocess.run([tool, "metric", "-g", "0", "-c", "--json"], capture_output=True, text=True,
                               timeout=30)
            d = json.loads(p.stdout)
            g = d[0] if isinstance(d, list) else d
            if isinstance(g, dict) and "gpu_data" in g:
                g = g["gpu_data"][0]
            clk = g["clock"]
            vals = [v["clk"]["value"] for k, v in clk.items()
                    if k.startswith("gfx") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
            if vals:
                readings.append(vals)
    except (subprocess.SubprocessError, ValueError, KeyError, IndexError, TypeError) as e:
        err = f"amd-smi: {e}"
    stop.set()
    th.join()
    torch.cuda.synchronize()
    if err is not None:
        return None, err
    if not readings:
        return None, "no gfx clock in amd-smi output"
    flat = [v for r in readings for v in r]
    return sum(flat) / len(flat), readings


# --- parity in the same run, and the CPU baseline ------------------------------------
def parity_and_cpu_baseline(A, B, C0, alpha, beta, C_gpu, exact: bool, kind16, single_core_s: float):
    """Every element of the GPU result against the float64 oracle on the same
    operands (A, B as they enter the product; 16-bit patterns decoded exactly).
    Returns (parity, cpu_baseline): the oracle's run on all host cores over the
    whole product is the CPU baseline, and one thread on the first rows (about
    `single_core_s` seconds) is a per-core reference."""
    import numpy as np

    import oracle

    if kind16:
        A = oracle.decode_16(A, kind16)
        B = oracle.decode_16(B, kind16)
    M, K = A.shape
    N = B.shape[1]
    cores = oracle.num_threads()
    t0 = time.perf_counter()
    Cref, absab = oracle.sgemm_ref(A, B, alpha, beta, C0)
    dt = time.perf_counter() - t0
    if exact:
        ok, info = oracle.check_bitexact(C_gpu, Cref)
        parity = {"ok": ok, "elements": int(M * N), "check": "bit-exact (integer-valued inputs)",
                  "n_bad": info["n_bad"]}
    else:
        ok, info = oracle.check_within_bound(C_gpu, Cref, oracle.error_bound(absab, alpha, beta, C0))
        parity = {"ok": ok, "elements": int(M * N),
                  "check": "|C - Cref| <= 2e-5 (|alpha| |A||B| + |beta| |C0|)",
                  "n_bad": info["n_bad"], "max_err_over_bound": round(info.get("max_err_over_bound", 0.0), 6)}
    if "first_bad_index" in info:
        parity["first_bad_index"] = list(info["first_bad_index"])
    del Cref, absab
    oracle.set_num_threads(1)
    try:
        r1 = int(min(M, max(1, single_core_s / max(dt / M * cores, 1e-9))))
        t0 = time.perf_counter()
        oracle.sgemm_ref(A[:r1], B, alpha, beta, None if C0 is None else C0[:r1])
        dt1 = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(cores)
    base = {
        "value": round(gemm_flops(M, N, K) / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"the whole {M}x{N}x{K} product ({M * N} outputs, float64 accumulation, "
                  f"{dt:.1f} s; the run that checks the GPU result)",
        "single_core": {"value": round(gemm_flops(r1, N, K) / dt1 / 1e12, 6), "unit": "TFLOP/s",
                        "sample": f"rows 0..{r1 - 1} of the same product on one thread ({dt1:.1f} s)"},
    }
    return parity, base


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
    ap.add_argument("--prewarm-seconds", type=float, default=0.6,
                    help="back-to-back launches before anything is counted (the GPU starts in a "
                         "low-power state)")
    ap.add_argument("--round-seconds", type=float, default=0.5,
                    help="length of each of the three interleaved timing rounds (0: none)")
    ap.add_argument("--single-core-seconds", type=float, default=1.5,
                    help="approximate time of the one-thread oracle reference")
    ap.add_argument("--plan", default=None, metavar="CONFIG[:GROUP[:SPLITS]]",
                    help="run one MFMA plan through sgemm_f32_ex_config instead of the automatic choice")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle: no parity check and no CPU baseline (profiling runs)")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the rocBLAS / torch timings and the clock reading")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the shader-clock reading, which starts amd-smi as a child program "
                         "(runs under a profiler that preloads itself into every process)")
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
    forced = None
    if args.plan:
        parts = [int(v) for v in args.plan.split(":")]
        forced = (parts + [8, 1][len(parts) - 1:])[:3]
        if kind16:
            sys.exit("--plan applies to the FP32 path only")
        chosen = sg.MFMA_TUNED
        plan = {"config": sg.sgemm_f32_config_name(forced[0]), "group_m": forced[1], "splits": forced[2],
                "forced": True}
    elif variant in (0, sg.MFMA_TUNED):
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
        elif forced is not None:
            st = sg.sgemm_f32_ex_config(forced[0], forced[1], forced[2], ta, tb, w.M, w.N, w.K, w.alpha,
                                        dA.data_ptr(), lda, b.data_ptr(), ldb, w.beta, dC.data_ptr(), ldc, s_handle)
        elif ta or tb:
            st = sg.sgemm_f32_ex_variant(variant, ta, tb, w.M, w.N, w.K, w.alpha, dA.data_ptr(), lda,
                                         b.data_ptr(), ldb, w.beta, dC.data_ptr(), ldc, s_handle)
        else:
            st = sg.sgemm_f32_variant(variant, w.M, w.N, w.K, w.alpha, dA.data_ptr(), lda,
                                      b.data_ptr(), ldb, w.beta, dC.data_ptr(), ldc, s_handle)
        if st != 0:
            raise RuntimeError(f"sgemm_f32 returned {st}")

    torch.cuda.synchronize(dev)
    prewarm_s = prewarm(torch, stream, step, args.prewarm_seconds) if args.prewarm_seconds > 0 else 0.0
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize(dev)

    # The timed region: the steps back to back between one pair of HIP events
    # on the kernel's stream.  On this GPU a timing event recorded between two
    # kernels costs several microseconds of GPU time (about 7 us per pair,
    # measured at 1024^3), so events around every launch would slow a short
    # kernel down by a large fraction; the pages' per-launch statistic is taken
    # in a pass of its own right after (kernel_median_last_3q_ms).
    region_start = torch.cuda.Event(enable_timing=True)
    region_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        region_start.record(stream)
        for i in range(args.steps):
            step()
        region_end.record(stream)
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    region_ms = region_start.elapsed_time(region_end)
    # Each launch between its own pair of events (the pages' method), as many
    # launches as the timed region, not counted in the value.
    kern_ms = event_launches(torch, stream, step, args.steps)

    elapsed = t1 - t0
    flops = gemm_flops(w.M, w.N, w.K)
    value = flops * args.steps / elapsed / 1e12
    kern_avg_s = region_ms / args.steps / 1e3
    kern_med_s = median_last_three_quarters(kern_ms) / 1e3
    achieved = flops / kern_avg_s / 1e12

    peak = PEAK_16BIT_TFLOPS if kind16 else PEAK_FP32_TFLOPS
    memory_bound = arithmetic_intensity(w.M, w.N, w.K, w.beta != 0) < peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    min_bytes = gemm_min_bytes(w.M, w.N, w.K, w.beta != 0)
    if kind16 and not memory_bound:
        roofline = {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4)}
    elif memory_bound:
        ach_gbs = min_bytes / kern_avg_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(ach_gbs, 2), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(ach_gbs / PEAK_HBM_GBS, 4)}
    else:
        # The VALU comparison kernel is bound by the vector FP32 rate; every
        # other kernel by the FP32 matrix-core rate (the same datasheet number).
        bound = "alu" if chosen == sg.VALU else "mfma"
        roofline = {"bound": bound, "achieved": round(achieved, 3), "peak": PEAK_FP32_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_TFLOPS, 4)}
    headline_kernel = (w.name == workloads.HEADLINE and variant == 0 and forced is None and not (ta or tb)
                       and not kind16 and len(dBs) == 1)
    roofline["traffic"] = measured_traffic() if headline_kernel else None
    roofline["kernel_avg_ms"] = round(kern_avg_s * 1e3, 5)
    roofline["kernel_median_last_3q_ms"] = round(kern_med_s * 1e3, 5)
    roofline["timing"] = ("kernel_avg_ms: one pair of HIP events around the timed steps on the kernel's "
                          "stream, divided by the steps; kernel_median_last_3q_ms: a second pass with each "
                          "launch between its own pair of events (adds several us of GPU time per launch)")

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
        "prewarm_s": round(prewarm_s, 3),
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
    if memory_bound:
        out["gb_per_s"] = round(min_bytes * args.steps / elapsed / 1e9, 2)
    if not args.no_context:
        if kind16:
            calls, notes = library_calls16(torch, w, ta, tb, dA, dBs, kind16)
        else:
            calls, notes = library_calls(torch, w, ta, tb, dA, lda, dBs, ldb, C0, stream)
        calls = {"this_library": step, **calls}
        est = {"this_library": kern_avg_s * 1e3}
        for name, call in calls.items():
            if name != "this_library":
                ms = event_launches(torch, stream, call, 5)
                est[name] = float(np.median(ms))
        if args.round_seconds > 0:
            res = timed_rounds(torch, stream, calls, est, args.round_seconds)
            ctx = {}
            for name, r in res.items():
                med = sorted(r["rounds_ms"])[len(r["rounds_ms"]) // 2]
                entry = {"value": round(flops / (med * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
                         "rounds": [round(flops / (m * 1e-3) / 1e12, 3) for m in r["rounds_ms"]],
                         "mean_launch": round(flops / (float(np.mean(r["all_ms"])) * 1e-3) / 1e12, 3),
                         "launches": len(r["all_ms"])}
                entry.update(notes.get(name, {}))
                ctx[name] = entry
            for name, note in notes.items():
                if name not in ctx:
                    ctx[name] = note
            out["context"] = {"method": "three interleaved rounds of back-to-back launches, each "
                                        f"about {args.round_seconds} s; per round the median of the "
                                        "last three quarters; value = median over rounds",
                              **ctx}
        if args.no_clock:
            mhz, readings = None, "not read (--no-clock)"
        else:
            mhz, readings = gfx_clock_mhz(torch, step, stream, kern_avg_s)
        if mhz is not None:
            # 256 CUs x 4 matrix-core SIMDs x 64 FP32 FLOP per clock each.
            adj = 256 * 256 * mhz * 1e6 / 1e12
            out["clock"] = {"gfx_mhz": round(mhz, 1), "clock_adjusted_fp32_peak": round(adj, 2),
                            "frac_of_clock_adjusted_peak": None if kind16 else round(achieved / adj, 4),
                            "readings": readings}
            if kind16:
                # 16-bit inputs: 1024 FLOP per clock per SIMD (2.5 PFLOP/s at 2.4 GHz).
                adj16 = 256 * 4 * 1024 * mhz * 1e6 / 1e12
                out["clock"]["clock_adjusted_16bit_peak"] = round(adj16, 1)
                out["clock"]["frac_of_clock_adjusted_16bit_peak"] = round(achieved / adj16, 4)
        else:
            out["clock"] = {"gfx_mhz": None, "note": readings}
    failed = False
    if not args.no_cpu_baseline:
        # One more call on the initial C (beta != 0 reads it), with the first B
        # copy, checked element by element.
        if C0 is not None:
            dC.copy_(torch.from_numpy(C0).to(dev))
        else:
            dC.fill_(float("nan"))
        counter[0] = 0
        torch.cuda.synchronize(dev)
        with torch.cuda.stream(stream):
            step()
        torch.cuda.synchronize(dev)
        C_gpu = dC.cpu().numpy()
        parity, base = parity_and_cpu_baseline(A, B, C0, w.alpha, w.beta, C_gpu, w.dist == "int4", kind16,
                                               args.single_core_seconds)
        out["parity"] = parity
        out["cpu_baseline"] = base
        failed = not parity["ok"]
    print(json.dumps(out), flush=True)
    if failed:
        print("parity check FAILED: the timed result does not match the oracle", file=sys.stderr)
        sys.exit(3)


if __name__ == "__main__":
    main()
