"""The allocation-free entry point sgemm_f32_noalloc, through the C interface,
against sgemm_f32 on the same inputs: the same plan and kernels, so the same
bits, and within the oracle's bound (bit for bit against it on integer
inputs).  Each case runs two calls in a row on one stream, the second on a
smaller product, so the second reads a fixed scratch region that still holds
the first call's partial sums."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import check_full, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sg():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import fp32_sgemm_amd
    return fp32_sgemm_amd


def _inputs(M, N, K, dist, seed):
    w = workloads.custom(M, N, K, dist=dist, seed=seed, c0_dist="normal" if dist != "int4" else "int4")
    return workloads.make_inputs(w)


def _plan(sg, M, N, K):
    st, variant, config, group_m, splits = sg.sgemm_f32_ex_plan(0, 0, M, N, K, 1.0, 0x100000, K, 0x100000, N)
    assert st == 0
    return variant, config, splits


def _both(sg, A, B, C0, alpha, beta, stream):
    """C from sgemm_f32_noalloc and from sgemm_f32 on the same inputs."""
    M, K = A.shape
    N = B.shape[1]
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    c_init = torch.from_numpy(C0).cuda() if C0 is not None else torch.full((M, N), float("nan"), device="cuda:0")
    dC1, dC2 = c_init.clone(), c_init.clone()
    torch.cuda.synchronize()
    st1 = sg.sgemm_f32_noalloc(M, N, K, alpha, dA.data_ptr(), K, dB.data_ptr(), N, beta, dC1.data_ptr(), N,
                               stream.cuda_stream)
    st2 = sg.sgemm_f32(M, N, K, alpha, dA.data_ptr(), K, dB.data_ptr(), N, beta, dC2.data_ptr(), N,
                       stream.cuda_stream)
    torch.cuda.synchronize()
    return st1, st2, dC1.cpu().numpy(), dC2.cpu().numpy()


# (first, second) products: the second is smaller.  The automatic plans: the
# M <= 16 split (scratch), a tuned split-K plan (scratch), the 64x64
# direct-to-LDS grid (no scratch), the 4-byte-load tiles with K split (an
# odd row stride of B or A), and operands copied to aligned scratch rows
# before a 64x64 plan (odd row strides on a larger product), without and with
# a K split whose partials share the copies' scratch.
CASES = {
    "skinny": ((16, 4096, 4096), (8, 1000, 3000)),
    "splitk": ((512, 512, 8192), (256, 256, 4096)),
    "grid": ((1024, 1024, 1024), (256, 384, 512)),
    "unaligned": ((4096, 17, 4096), (1000, 33, 3001)),
    "packed": ((2047, 2047, 2047), (1500, 1600, 1999)),
    "packed_split": ((300, 3001, 4096), (512, 2047, 4096)),
}


@pytest.mark.parametrize("dist", ["uniform", "int4"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_noalloc_matches_sgemm_f32(sg, case, dist):
    s = torch.cuda.Stream()
    for idx, (M, N, K) in enumerate(CASES[case]):
        variant, config, splits = _plan(sg, M, N, K)
        say(f"[noalloc] {case} call {idx + 1}: {M}x{N}x{K} {dist} plan variant={variant} config={config} "
            f"splits={splits}")
        if case in ("splitk", "unaligned", "packed_split"):
            assert splits > 1, "the case needs a plan with a K split"
        A, B, C0 = _inputs(M, N, K, dist, 500 + 10 * idx + len(case))
        alpha, beta = (1.5, -0.5) if idx == 0 else (-1.0, 0.0)
        if beta == 0.0:
            C0 = None
        st1, st2, C1, C2 = _both(sg, A, B, C0, alpha, beta, s)
        assert st1 == 0 and st2 == 0
        assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32)), "noalloc differs from sgemm_f32"
        ok, info = check_full(C1, A, B, alpha, beta, C0, exact=(dist == "int4"))
        assert ok, info


def test_noalloc_refuses_a_plan_beyond_its_scratch(sg):
    """A plan whose split partials exceed the fixed region returns
    SGEMM_F32_ERR_SCRATCH and leaves C untouched; sgemm_f32 runs it."""
    M, K = 64, 2048
    N = None
    for n in (40000, 80000, 160000):
        variant, config, splits = _plan(sg, M, n, K)
        if splits > 1 and splits * M * n * 4 > sg.NOALLOC_SCRATCH_BYTES:
            N = n
            break
    if N is None:
        pytest.skip("no automatic plan of this shape class needs more scratch than the fixed region")
    say(f"[noalloc_refuse] {M}x{N}x{K} splits={splits}")
    A, B, _ = _inputs(M, N, K, "int4", 600)
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    dC = torch.full((M, N), 7.0, device="cuda:0")
    st = sg.sgemm_f32_noalloc(M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, dC.data_ptr(), N,
                              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == sg.ERR_SCRATCH
    assert torch.all(dC == 7.0)
    st = sg.sgemm_f32(M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, dC.data_ptr(), N,
                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    ok, info = check_full(dC.cpu().numpy(), A, B, 1.0, 0.0, None, exact=True)
    assert ok, info
