"""Seeded synthetic inputs for the FP32 GEMM workloads.

This module only draws random matrices.  It holds none of the GEMM arithmetic,
so both the GPU side (benchmark, GPU tests) and the oracle side (CPU checks) can
use it without sharing any of the method's code.

Workloads are square and rectangular row-major FP32 products with the shapes the
pages measure: 4092^3 ("Learn: Optimizing GEMM", section 2 table; "How a Matmul
Kernel Gets Fast", section 2), 4096^3 ("Writing a Fast Matmul in CUDA, Step by
Step", section "Step 1"), 1024^3 (same page, section "Size effects"), with
entries drawn uniformly from [-1, 1] as that page's correctness check does.

Conventions:
  * uniform[-1, 1] is drawn as 2*U[0,1) - 1 in float32, so values lie in [-1, 1);
  * "int4" draws integers uniformly from {-4, ..., 4} (inclusive) as float32;
  * "normal" is the standard normal N(0, 1) in float32;
  * every matrix has its own seed: 1000*cid + 0 for A, + 1 for B, + 2 for C0,
    with a CPU ``torch.Generator`` (deterministic across machines).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dist: str          # "uniform" | "int4" | "normal"
    alpha: float
    beta: float
    cid: int           # seed base: seeds are 1000*cid + {0: A, 1: B, 2: C0}
    c0_dist: str | None = None   # distribution of the initial C (None: C not read)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


WORKLOADS = {
    w.name: w for w in [
        Workload("square128", 128, 128, 128, "uniform", 1.0, 0.0, 1),
        Workload("square128_int", 128, 128, 128, "int4", 1.0, 0.0, 10),
        Workload("square1024", 1024, 1024, 1024, "uniform", 1.0, 0.0, 2),
        Workload("square4092", 4092, 4092, 4092, "uniform", 1.0, 0.0, 3),
        Workload("square4096_ab", 4096, 4096, 4096, "normal", 1.5, -0.5, 4, "normal"),
        Workload("square8192", 8192, 8192, 8192, "uniform", 1.0, 0.0, 51),
        Workload("skinny16x4096x4096", 16, 4096, 4096, "uniform", 1.0, 0.0, 52),
        Workload("wide4096x11008x512", 4096, 11008, 512, "uniform", 1.0, 0.0, 53),
    ]
}

HEADLINE = "square4096_ab"


def draw(shape, dist: str, seed: int, pad_cols: int = 0) -> np.ndarray:
    """One float32 matrix of ``shape`` drawn from ``dist`` with ``seed``.

    With ``pad_cols > 0`` the array has ``pad_cols`` extra columns (filled from
    the same stream) and the function returns the view of the first
    ``shape[1]`` columns, i.e. a matrix whose row stride exceeds its width.
    """
    rows, cols = int(shape[0]), int(shape[1])
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    full = (rows, cols + pad_cols)
    if dist == "uniform":
        t = torch.rand(full, generator=g, dtype=torch.float32) * 2.0 - 1.0
    elif dist == "int4":
        t = torch.randint(-4, 5, full, generator=g, dtype=torch.int32).to(torch.float32)
    elif dist == "normal":
        t = torch.randn(full, generator=g, dtype=torch.float32)
    elif dist == "ones":
        t = torch.ones(full, dtype=torch.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    arr = t.numpy()
    return arr[:, :cols] if pad_cols else arr


def make_inputs(w: Workload, pad: tuple[int, int, int] = (0, 0, 0)):
    """(A, B, C0) for a workload; C0 is None when the workload never reads C."""
    A = draw((w.M, w.K), w.dist, 1000 * w.cid + 0, pad[0])
    B = draw((w.K, w.N), w.dist, 1000 * w.cid + 1, pad[1])
    C0 = None
    if w.c0_dist is not None:
        C0 = draw((w.M, w.N), w.c0_dist, 1000 * w.cid + 2, pad[2])
    return A, B, C0


def custom(M: int, N: int, K: int, dist: str = "uniform", seed: int = 7,
           alpha: float = 1.0, beta: float = 0.0, c0_dist: str | None = None,
           name: str | None = None) -> Workload:
    """A workload of any shape (parity cases: ragged tails, tiny sizes)."""
    return Workload(name or f"custom{M}x{N}x{K}", M, N, K, dist, alpha, beta,
                    seed, c0_dist)


BF16 = 1
F16 = 2


def to_16bit(x: np.ndarray, kind: int) -> np.ndarray:
    """Stores float32 values in a 16-bit input format (kind 1 bfloat16, kind 2
    binary16), rounding to nearest even, as a uint16 array of bit patterns.
    Input preparation only: the conversion is torch's own."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    dt = torch.bfloat16 if kind == BF16 else torch.float16
    return t.to(dt).view(torch.int16).numpy().view(np.uint16)


def make_inputs_16bit(w: Workload, kind: int):
    """(A bits, B bits, C0) for the 16-bit-input form of a workload: the same
    draws as ``make_inputs``, A and B stored in the 16-bit format, C0 float32."""
    A, B, C0 = make_inputs(w)
    return to_16bit(A, kind), to_16bit(B, kind), C0
