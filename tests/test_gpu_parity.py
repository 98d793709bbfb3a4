"""GPU parity: the HIP library, called through its C interface, against the oracle.

Real-valued inputs must satisfy |C - Cref| <= 2e-5 * (|alpha|*(|A||B|)_ij +
|beta|*|C0_ij|) element by element; integer-valued inputs (exact in FP32) must
match bit for bit.  Sizes span several tiles with ragged tails; the full-size
workloads are checked element by element against the full oracle as well.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import check_full, run_lib, say, zero_sum_integers

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sg():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import fp32_sgemm_amd
    return fp32_sgemm_amd


GENERAL = ["auto", "mfma_large", "mfma_small", "valu", "mfma_scalar"]
VID = {"auto": 0, "mfma_large": 1, "mfma_small": 2, "valu": 3, "skinny": 4, "mfma_scalar": 5}

RAGGED = [(1, 1, 1), (2, 3, 5), (17, 31, 33), (63, 65, 127), (129, 127, 65),
          (300, 260, 70), (257, 129, 1000), (128, 128, 128), (64, 64, 32), (96, 200, 31),
          (33, 17, 1), (130, 70, 9)]


def _inputs(M, N, K, dist, seed, c0=True):
    w = workloads.custom(M, N, K, dist=dist, seed=seed, c0_dist=("normal" if dist != "int4" else "int4") if c0 else None)
    return workloads.make_inputs(w)


@pytest.mark.parametrize("variant", GENERAL)
@pytest.mark.parametrize("shape", RAGGED, ids=[f"{m}x{n}x{k}" for m, n, k in RAGGED])
def test_ragged_real(sg, variant, shape):
    M, N, K = shape
    say(f"[ragged_real] {variant} {shape}")
    A, B, C0 = _inputs(M, N, K, "uniform", 100 + M + N + K)
    st, C, _ = run_lib(sg, VID[variant], A, B, C0, 1.25, -0.5)
    assert st == 0
    ok, info = check_full(C, A, B, 1.25, -0.5, C0)
    assert ok, info


@pytest.mark.parametrize("variant", GENERAL)
@pytest.mark.parametrize("shape", RAGGED, ids=[f"{m}x{n}x{k}" for m, n, k in RAGGED])
def test_ragged_integer_bitexact(sg, variant, shape):
    M, N, K = shape
    say(f"[ragged_int] {variant} {shape}")
    A, B, C0 = _inputs(M, N, K, "int4", 200 + M + N + K)
    st, C, _ = run_lib(sg, VID[variant], A, B, C0, 1.5, -0.5)
    assert st == 0
    ok, info = check_full(C, A, B, 1.5, -0.5, C0, exact=True)
    assert ok, info


SKINNY = [(1, 1, 1), (16, 16, 16), (16, 4096, 64), (3, 33, 100), (16, 100, 4099),
          (7, 257, 513), (16, 16, 17), (12, 64, 2000), (5, 130, 777), (16, 65, 1000),
          (1, 1, 5000), (16, 4096, 300), (16, 2050, 8191),
          # 16 < M <= 32: two blocks of 16 rows of A per work-group
          (17, 4096, 4096), (24, 100, 4099), (32, 2050, 1000), (20, 130, 777), (32, 16, 17),
          # 5 and 7 batches per wave (three in flight), and grids of more
          # than 64 strips (two in flight)
          (16, 4096, 2560), (31, 4093, 3584), (27, 64, 128), (17, 4160, 1000), (16, 8200, 3000), (9, 4097, 5)]


@pytest.mark.parametrize("variant", ["skinny", "auto", "mfma_scalar", "valu"])
@pytest.mark.parametrize("shape", SKINNY, ids=[f"{m}x{n}x{k}" for m, n, k in SKINNY])
def test_skinny_shapes(sg, variant, shape):
    M, N, K = shape
    say(f"[skinny] {variant} {shape}")
    A, B, C0 = _inputs(M, N, K, "uniform", 300 + M + N + K)
    st, C, _ = run_lib(sg, VID[variant], A, B, C0, -0.75, 2.0)
    assert st == 0
    ok, info = check_full(C, A, B, -0.75, 2.0, C0)
    assert ok, info
    Ai, Bi, _ = _inputs(M, N, K, "int4", 400 + M + N + K, c0=False)
    st, C, _ = run_lib(sg, VID[variant], Ai, Bi, None, 1.0, 0.0)
    assert st == 0
    ok, info = check_full(C, Ai, Bi, 1.0, 0.0, None, exact=True)
    assert ok, info


# Grids with edge tiles through the automatic plan: 64x64 direct-to-LDS tiles
# (M, N multiples of 4), one round of 128x128 ones, and a K split where the
# 64x64 grid spreads unevenly (also with odd M).
AUTO_EDGE = [(500, 2000, 4096), (1020, 1020, 1020), (2044, 2044, 2044), (700, 900, 3000), (100, 5000, 2048),
             (131, 6000, 2048), (1001, 1500, 2048)]


@pytest.mark.parametrize("shape", AUTO_EDGE, ids=[f"{m}x{n}x{k}" for m, n, k in AUTO_EDGE])
def test_auto_plans_with_edge_tiles(sg, shape):
    M, N, K = shape
    say(f"[auto_edge] {shape}")
    A, B, C0 = _inputs(M, N, K, "uniform", 90 + M)
    st, C, _ = run_lib(sg, VID["auto"], A, B, C0, 1.25, -0.5)
    assert st == 0
    ok, info = check_full(C, A, B, 1.25, -0.5, C0)
    assert ok, info
    Ai, Bi, _ = _inputs(M, N, K, "int4", 95 + M, c0=False)
    st, C, _ = run_lib(sg, VID["auto"], Ai, Bi, None, -1.0, 0.0)
    assert st == 0
    ok, info = check_full(C, Ai, Bi, -1.0, 0.0, None, exact=True)
    assert ok, info


# N not a multiple of 4 with B as given (16-byte groups straddle the N edge):
# K split over a grid of one round; with an odd row stride of B as well, B is
# first copied to aligned rows and the split partials share that scratch.
STRADDLE = [(512, 2047, 4096, 2048), (300, 3001, 4096, None), (2048, 1023, 2048, 1024)]


@pytest.mark.parametrize("case", STRADDLE, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in STRADDLE])
def test_auto_straddling_edge_split(sg, case):
    M, N, K, ldb = case
    say(f"[straddle] {case}")
    plan = sg.sgemm_f32_ex_plan(0, 0, M, N, K, 1.0, 256, K, 256, ldb or N)
    assert plan[4] > 1, plan
    A, B, C0 = _inputs(M, N, K, "uniform", 97 + M)
    st, C, _ = run_lib(sg, VID["auto"], A, B, C0, 1.25, -0.5, ldb=ldb)
    assert st == 0
    ok, info = check_full(C, A, B, 1.25, -0.5, C0)
    assert ok, info
    Ai, Bi, _ = _inputs(M, N, K, "int4", 98 + M, c0=False)
    st, C, _ = run_lib(sg, VID["auto"], Ai, Bi, None, -1.0, 0.0, ldb=ldb)
    assert st == 0
    ok, info = check_full(C, Ai, Bi, -1.0, 0.0, None, exact=True)
    assert ok, info


# Row strides that 16-byte loads cannot take, on grids of few tiles: the
# automatic plan splits K over the 4-byte-load tiles.
UNALIGNED_FEW = [(4096, 17, 4096, None, None), (1000, 33, 3001, None, None), (300, 100, 2001, 2003, None),
                 (130, 250, 5000, None, 251), (64, 64, 256, 257, None)]


@pytest.mark.parametrize("case", UNALIGNED_FEW, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in UNALIGNED_FEW])
def test_unaligned_few_tiles_split(sg, case):
    M, N, K, lda, ldb = case
    say(f"[unaligned_split] {case}")
    A, B, C0 = _inputs(M, N, K, "uniform", 40 + M)
    st, C, _ = run_lib(sg, VID["auto"], A, B, C0, 1.25, -0.5, lda=lda, ldb=ldb)
    assert st == 0
    ok, info = check_full(C, A, B, 1.25, -0.5, C0)
    assert ok, info
    Ai, Bi, _ = _inputs(M, N, K, "int4", 50 + M, c0=False)
    st, C, _ = run_lib(sg, VID["auto"], Ai, Bi, None, -1.0, 0.0, lda=lda, ldb=ldb)
    assert st == 0
    ok, info = check_full(C, Ai, Bi, -1.0, 0.0, None, exact=True)
    assert ok, info
    plan = sg.sgemm_f32_ex_plan(0, 0, M, N, K, 1.0, 256, lda or K, 256, ldb or N)
    assert plan[1] == sg.MFMA_SCALAR and (plan[4] > 1) == (K >= 512), plan


# Odd row strides on larger products: the operands that 16-byte loads cannot
# take are copied into aligned scratch rows first (A, B or both).
PACKED = [(2047, 2047, 2047, None, None), (2048, 2048, 2047, None, 2048), (1300, 2001, 1999, 2000, None),
          (1500, 1600, 1999, None, 1601)]


@pytest.mark.parametrize("case", PACKED, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in PACKED])
def test_unaligned_operands_packed(sg, case):
    M, N, K, lda, ldb = case
    say(f"[packed] {case}")
    plan = sg.sgemm_f32_ex_plan(0, 0, M, N, K, 1.0, 256, lda or K, 256, ldb or N)
    assert plan[1] != sg.MFMA_SCALAR, plan
    A, B, C0 = _inputs(M, N, K, "uniform", 60 + M)
    st, C, _ = run_lib(sg, VID["auto"], A, B, C0, 1.25, -0.5, lda=lda, ldb=ldb)
    assert st == 0
    ok, info = check_full(C, A, B, 1.25, -0.5, C0)
    assert ok, info
    # The same plan on aligned copies gives the same bits.
    dA = torch.from_numpy(np.pad(A, ((0, 0), (0, (-K) % 4)))).cuda()
    dB = torch.from_numpy(np.pad(B, ((0, 0), (0, (-N) % 4)))).cuda()
    dC = torch.from_numpy(C0).cuda()
    st = sg.sgemm_f32_ex_config(plan[2], plan[3], plan[4], 0, 0, M, N, K, 1.25, dA.data_ptr(), dA.shape[1],
                                dB.data_ptr(), dB.shape[1], -0.5, dC.data_ptr(), N,
                                torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert np.array_equal(dC.cpu().numpy().view(np.uint32), C.view(np.uint32))
    Ai, Bi, _ = _inputs(M, N, K, "int4", 70 + M, c0=False)
    st, C, _ = run_lib(sg, VID["auto"], Ai, Bi, None, -1.0, 0.0, lda=lda, ldb=ldb)
    assert st == 0
    ok, info = check_full(C, Ai, Bi, -1.0, 0.0, None, exact=True)
    assert ok, info


@pytest.mark.parametrize("variant", GENERAL + ["skinny"])
def test_beta_zero_ignores_nan_c(sg, variant):
    for M in ((16, 27) if variant == "skinny" else (150,)):   # one and two blocks of 16 rows
        A, B, _ = _inputs(M, 140, 90, "uniform", 11, c0=False)
        st, C, _ = run_lib(sg, VID[variant], A, B, None, 1.0, 0.0, c_fill=np.nan)
        assert st == 0
        assert np.all(np.isfinite(C))
        ok, info = check_full(C, A, B, 1.0, 0.0, None)
        assert ok, info


@pytest.mark.parametrize("variant", GENERAL + ["skinny"])
def test_guard_bands_untouched(sg, variant):
    """C lives inside a larger buffer with row stride ldc > N and an offset:
    every float outside the M x N window keeps its sentinel bits."""
    M = 13 if variant == "skinny" else 133
    N, K, ldc, off = 75, 41, 83, 4
    A, B, C0 = _inputs(M, N, K, "uniform", 12)
    st, C, Cbuf = run_lib(sg, VID[variant], A, B, C0, 1.0, 1.0, ldc=ldc, offs=(0, 0, off))
    assert st == 0
    ok, info = check_full(C, A, B, 1.0, 1.0, C0)
    assert ok, info
    mask = np.ones(Cbuf.shape, bool)
    for i in range(M):
        mask[off + i * ldc: off + i * ldc + N] = False
    assert np.all(Cbuf[mask].view(np.uint32) == np.float32(-7.25).view(np.uint32))


@pytest.mark.parametrize("variant", ["auto", "mfma_scalar", "valu", "skinny"])
def test_odd_strides_and_misaligned_pointers(sg, variant):
    M = 9 if variant == "skinny" else 140
    N, K = 97, 61
    A, B, C0 = _inputs(M, N, K, "uniform", 13)
    st, C, _ = run_lib(sg, VID[variant], A, B, C0, 0.5, 0.25, lda=K + 1, ldb=N + 3, ldc=N + 2,
                       offs=(1, 3, 1))
    assert st == 0
    ok, info = check_full(C, A, B, 0.5, 0.25, C0)
    assert ok, info


def test_vector_variants_refuse_misaligned(sg):
    A, B, C0 = _inputs(64, 64, 64, "uniform", 14)
    for v in ("mfma_large", "mfma_small"):
        st, _, _ = run_lib(sg, VID[v], A, B, C0, 1.0, 0.0, lda=65)
        assert st == sg.ERR_NOT_APPLICABLE
        st, _, _ = run_lib(sg, VID[v], A, B, C0, 1.0, 0.0, offs=(1, 0, 0))
        assert st == sg.ERR_NOT_APPLICABLE
    st, _, _ = run_lib(sg, VID["skinny"], A, B, C0, 1.0, 0.0)
    assert st == sg.ERR_NOT_APPLICABLE


def test_alpha_zero_and_k_zero(sg):
    M, N, K = 70, 90, 30
    rng = np.random.default_rng(1)
    C0 = rng.standard_normal((M, N)).astype(np.float32)
    A = np.full((M, K), np.nan, np.float32)
    B = np.full((K, N), np.nan, np.float32)
    st, C, _ = run_lib(sg, 0, A, B, C0, 0.0, -0.5)
    assert st == 0
    assert np.array_equal(C, (np.float32(-0.5) * C0))
    A0 = np.zeros((M, 0), np.float32)
    B0 = np.zeros((0, N), np.float32)
    st, C, _ = run_lib(sg, 0, A0, B0, C0, 2.0, 3.0)
    assert st == 0
    assert np.array_equal(C, np.float32(3.0) * C0)
    st, C, _ = run_lib(sg, 0, A0, B0, None, 2.0, 0.0, c_fill=np.nan)
    assert st == 0
    assert np.array_equal(C, np.zeros((M, N), np.float32))
    st, C, _ = run_lib(sg, 0, A, B, C0, 0.0, 1.0)
    assert st == 0 and np.array_equal(C, C0)


def test_empty_output_is_noop(sg):
    A, B, _ = _inputs(0, 5, 7, "uniform", 15, c0=False)
    st, C, _ = run_lib(sg, 0, A, B, None, 1.0, 0.0)
    assert st == 0 and C.shape == (0, 5)
    A, B, _ = _inputs(5, 0, 7, "uniform", 15, c0=False)
    st, C, _ = run_lib(sg, 0, A, B, None, 1.0, 0.0)
    assert st == 0 and C.shape == (5, 0)


def test_invalid_arguments(sg):
    dC = torch.zeros(16, device="cuda:0")
    p = dC.data_ptr()
    assert sg.sgemm_f32(-1, 2, 2, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == 1
    assert sg.sgemm_f32(2, -1, 2, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == 2
    assert sg.sgemm_f32(2, 2, -1, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == 3
    assert sg.sgemm_f32(2, 2, 2, 1.0, 0, 2, p, 2, 0.0, p, 2, 0) == 5
    assert sg.sgemm_f32(2, 2, 3, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == 6
    assert sg.sgemm_f32(2, 2, 2, 1.0, p, 2, 0, 2, 0.0, p, 2, 0) == 7
    assert sg.sgemm_f32(2, 3, 2, 1.0, p, 2, p, 2, 0.0, p, 3, 0) == 8
    assert sg.sgemm_f32(2, 2, 2, 1.0, p, 2, p, 2, 0.0, 0, 2, 0) == 10
    assert sg.sgemm_f32(2, 3, 2, 1.0, p, 2, p, 3, 0.0, p, 2, 0) == 11
    assert sg.sgemm_f32_variant(99, 2, 2, 2, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == sg.ERR_VARIANT
    torch.cuda.synchronize()
    assert torch.all(dC == 0)


@pytest.mark.parametrize("variant", GENERAL + ["skinny"])
def test_repeat_runs_bitwise_identical(sg, variant):
    M = 16 if variant == "skinny" else 700
    N, K = 900, 1100
    A, B, C0 = _inputs(M, N, K, "uniform", 16)
    st1, C1, _ = run_lib(sg, VID[variant], A, B, C0, 1.0, 0.5)
    st2, C2, _ = run_lib(sg, VID[variant], A, B, C0, 1.0, 0.5)
    assert st1 == 0 and st2 == 0
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))


def test_skinny_concurrent_streams(sg):
    """Two M <= 16 products with split reductions in flight on two streams at
    once: each call's scratch memory is its own."""
    M, N, K = 16, 2048, 4096
    A1, B1, _ = _inputs(M, N, K, "uniform", 31, c0=False)
    A2, B2, _ = _inputs(M, N, K, "uniform", 32, c0=False)
    d = [torch.from_numpy(x).cuda() for x in (A1, B1, A2, B2)]
    C1 = torch.zeros(M, N, device="cuda:0")
    C2 = torch.zeros(M, N, device="cuda:0")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        st1 = sg.sgemm_f32_variant(4, M, N, K, 1.0, d[0].data_ptr(), K, d[1].data_ptr(), N, 0.0,
                                   C1.data_ptr(), N, s1.cuda_stream)
        st2 = sg.sgemm_f32_variant(4, M, N, K, 1.0, d[2].data_ptr(), K, d[3].data_ptr(), N, 0.0,
                                   C2.data_ptr(), N, s2.cuda_stream)
        assert st1 == 0 and st2 == 0
    torch.cuda.synchronize()
    ok, info = check_full(C1.cpu().numpy(), A1, B1, 1.0, 0.0, None)
    assert ok, info
    ok, info = check_full(C2.cpu().numpy(), A2, B2, 1.0, 0.0, None)
    assert ok, info


def test_scratch_sizes_and_host_threads(sg):
    """Products of different sizes in a row on one stream (its cached scratch
    block grows in stream order), and host threads calling on their own
    streams at the same time, which never share a block."""
    import threading
    cases = [(256, 256, 4096, 41), (512, 512, 8192, 42), (256, 256, 4096, 43)]
    data = []
    for M, N, K, seed in cases:
        A, B, _ = _inputs(M, N, K, "uniform", seed, c0=False)
        data.append((M, N, K, A, B, torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(),
                     torch.zeros(M, N, device="cuda:0")))
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    # configuration 4 (64x64, two slices in flight) with 8 K splits: 8*M*N floats of partials
    for M, N, K, _, _, dA, dB, dC in data:
        say(f"[scratch_sizes] {M}x{N}x{K} splits 8")
        assert sg.sgemm_f32_ex_config(4, 8, 8, 0, 0, M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0,
                                      dC.data_ptr(), N, s.cuda_stream) == 0
    torch.cuda.synchronize()
    for M, N, K, A, B, _, _, dC in data:
        ok, info = check_full(dC.cpu().numpy(), A, B, 1.0, 0.0, None)
        assert ok, info

    errors = []

    def worker(idx):
        M, N, K, A, B, dA, dB, _ = data[idx]
        st = torch.cuda.Stream()
        out = torch.zeros(M, N, device="cuda:0")
        for _ in range(4):
            rc = sg.sgemm_f32_ex_config(4, 8, 8, 0, 0, M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0,
                                        out.data_ptr(), N, st.cuda_stream)
            if rc != 0:
                errors.append(rc)
        st.synchronize()
        ok, info = check_full(out.cpu().numpy(), A, B, 1.0, 0.0, None)
        if not ok:
            errors.append(info)

    say("[scratch_threads] three host threads, three streams")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(3)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors


def test_scratch_cache_many_streams_and_large_requests(sg):
    """Eager calls keep a scratch block per stream for up to 8 streams, each
    block at most 64 MiB: here 11 streams have split plans in flight at once
    (the streams past the cache take stream-ordered pool memory per call), and
    one stream with a cached block also runs a product whose partial sums need
    75.5 MB (pool memory) between two that fit its block.  Every result is
    checked against the oracle."""
    small, big = (256, 256, 4096), (1536, 1536, 4096)
    streams = [torch.cuda.Stream() for _ in range(11)]
    jobs = []
    for i, st in enumerate(streams):
        M, N, K = small
        A, B, _ = _inputs(M, N, K, "uniform", 50 + i, c0=False)
        jobs.append((st, M, N, K, A, B, torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(),
                     torch.zeros(M, N, device="cuda:0")))
    M, N, K = big
    A, B, _ = _inputs(M, N, K, "uniform", 70, c0=False)
    big_job = (streams[0], M, N, K, A, B, torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(),
               torch.zeros(M, N, device="cuda:0"))
    torch.cuda.synchronize()

    def launch(job):
        st, M, N, K, _, _, dA, dB, dC = job
        # configuration 4 (64x64, two slices in flight) with 8 K splits: 8*M*N floats of partials
        return sg.sgemm_f32_ex_config(4, 8, 8, 0, 0, M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0,
                                      dC.data_ptr(), N, st.cuda_stream)

    say("[scratch_cache] 11 streams, then 75.5 MB of partials on the first")
    for _ in range(2):
        for job in jobs:
            assert launch(job) == 0
    assert launch(big_job) == 0
    assert launch(jobs[0]) == 0
    torch.cuda.synchronize()
    for _, M, N, K, A, B, _, _, dC in jobs + [big_job]:
        ok, info = check_full(dC.cpu().numpy(), A, B, 1.0, 0.0, None)
        assert ok, (M, N, K, info)


def test_non_default_stream_ordering(sg):
    """Work queued before the call on a side stream is seen by the kernel."""
    M, N, K = 300, 400, 500
    A, B, _ = _inputs(M, N, K, "uniform", 17, c0=False)
    s = torch.cuda.Stream()
    dA = torch.from_numpy(A).cuda()
    dB = torch.from_numpy(B).cuda()
    dC = torch.empty(M, N, device="cuda:0")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        dC.fill_(1.0)            # queued on s before the GEMM
        dA2 = dA * 2.0           # also on s
        st = sg.sgemm_f32(M, N, K, 0.5, dA2.data_ptr(), K, dB.data_ptr(), N, 1.0,
                          dC.data_ptr(), N, s.cuda_stream)
    s.synchronize()
    assert st == 0
    C = dC.cpu().numpy()
    ones = np.ones((M, N), np.float32)
    A2 = (A * np.float32(2.0)).astype(np.float32)
    ok, info = check_full(C, A2, B, 0.5, 1.0, ones)
    assert ok, info


# ---------------------------------------------------------------------------
# The named workloads at their full sizes, through sgemm_f32 (the launch the
# benchmark times), every element against the full oracle.
# ---------------------------------------------------------------------------
WORKLOAD_NAMES = ["square128", "square128_int", "square1024", "skinny16x4096x4096",
                  "square4092", "square4096_ab", "square8192", "wide4096x11008x512"]


def _run_workload(sg, w, dist=None):
    if dist is not None:
        w = workloads.Workload(w.name + "_int", w.M, w.N, w.K, dist, w.alpha, w.beta, w.cid + 900,
                               "int4" if w.c0_dist else None)
    A, B, C0 = workloads.make_inputs(w)
    st, C, _ = run_lib(sg, 0, A, B, C0, w.alpha, w.beta, c_fill=np.nan)
    assert st == 0
    return w, A, B, C0, C


@pytest.mark.parametrize("name", WORKLOAD_NAMES)
def test_workload_full_oracle(sg, name):
    w = workloads.WORKLOADS[name]
    say(f"[workload_full] {name} {w.M}x{w.N}x{w.K} alpha={w.alpha} beta={w.beta}")
    w, A, B, C0, C = _run_workload(sg, w)
    ok, info = check_full(C, A, B, w.alpha, w.beta, C0, exact=(w.dist == "int4"))
    say(f"[workload_full] {name} {info}")
    assert ok, info


@pytest.mark.parametrize("name", ["square4096_ab", "square4092"])
def test_workload_integer_bitexact_full(sg, name):
    """Integer-valued inputs of the full shape: every partial sum stays below
    2**24, so the GPU result is exact and must match bit for bit everywhere."""
    w = workloads.WORKLOADS[name]
    say(f"[workload_int] {name}")
    w, A, B, C0, C = _run_workload(sg, w, dist="int4")
    ok, info = check_full(C, A, B, w.alpha, w.beta, C0, exact=True)
    assert ok, info


@pytest.mark.parametrize("variant", GENERAL + ["skinny"])
def test_negative_alpha_zero_sums_bitexact(sg, variant):
    """alpha < 0, beta = 0: exactly zero sums come out as alpha * (+0) = -0,
    the oracle's value; every other entry is exact as well (integer inputs)."""
    M = 16 if variant == "skinny" else 150
    N, K = 140, 90
    A, B = zero_sum_integers(M, N, K, 70)
    st, C, _ = run_lib(sg, VID[variant], A, B, None, -1.0, 0.0, c_fill=np.nan)
    assert st == 0
    assert np.all(np.signbit(C[1, :])) and np.all(C[1, :] == 0)
    ok, info = check_full(C, A, B, -1.0, 0.0, None, exact=True)
    assert ok, info


# ---------------------------------------------------------------------------
# Degenerate and limit cases.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ["auto", "mfma_scalar", "valu", "skinny"])
def test_nan_and_inf_propagate(sg, variant):
    """IEEE propagation: a NaN row of A makes that row of C NaN, an infinite
    column of B (with nonzero A entries of both signs) makes that column of C
    non-finite; every other entry is unaffected and within the bound."""
    M = 9 if variant == "skinny" else 140
    N, K = 70, 33
    A, B, C0 = _inputs(M, N, K, "uniform", 60)
    A = A.copy(); B = B.copy()
    A[3, :] = np.nan
    B[:, 5] = np.inf
    st, C, _ = run_lib(sg, VID[variant], A, B, C0, 1.0, 0.5)
    assert st == 0
    assert np.all(np.isnan(C[3, :]))
    assert not np.any(np.isfinite(C[:, 5]))
    keep_r = np.array([i for i in range(M) if i != 3])
    keep_c = np.array([j for j in range(N) if j != 5])
    Cref, absab = oracle.sgemm_ref(A, B, 1.0, 0.5, C0)
    sub = np.ix_(keep_r, keep_c)
    ok, info = oracle.check_within_bound(C[sub], Cref[sub], oracle.error_bound(absab[sub], 1.0, 0.5, C0[sub]))
    assert ok, info


def test_leading_dimension_past_32bit_offsets(sg):
    """lda so large that 128 rows of A span more than 2 GiB: the 16-byte-load
    kernels cannot address a slice with 32-bit offsets, the automatic choice
    falls back to the 4-byte-load kernel, and the forced vector variants
    refuse."""
    M, N, K = 130, 70, 60
    lda = (1 << 31) // 4 // 127 + 8          # multiple of 4, 127 * lda * 4 > 2^31
    A, B, C0 = _inputs(M, N, K, "int4", 61)
    assert sg.sgemm_f32_select(M, N, K, 1.0, 0x100000, lda, 0x100000, N) == sg.MFMA_SCALAR
    say(f"[huge_lda] lda={lda} ({M * lda * 4 / 2**30:.2f} GiB for A)")
    st, C, _ = run_lib(sg, 0, A, B, C0, 1.0, 1.0, lda=lda)
    assert st == 0
    ok, info = check_full(C, A, B, 1.0, 1.0, C0, exact=True)
    assert ok, info
    st, _, _ = run_lib(sg, VID["mfma_large"], A, B, C0, 1.0, 1.0, lda=lda)
    assert st == sg.ERR_NOT_APPLICABLE
    torch.cuda.empty_cache()


def test_c_leading_dimension_past_32bit_offsets(sg):
    """ldc so large that 128 rows of C span more than 2 GiB: edge tiles write C
    through guarded pointers instead of a buffer resource."""
    M, N, K = 130, 70, 64
    ldc = (1 << 31) // 4 // 127 + 8
    A, B, C0 = _inputs(M, N, K, "int4", 62)
    say(f"[huge_ldc] ldc={ldc} ({M * ldc * 4 / 2**30:.2f} GiB for C)")
    st, C, Cbuf = run_lib(sg, VID["mfma_large"], A, B, C0, 1.0, -1.0, ldc=ldc)
    assert st == 0
    ok, info = check_full(C, A, B, 1.0, -1.0, C0, exact=True)
    assert ok, info
    del Cbuf
    torch.cuda.empty_cache()


# Shapes for which the automatic choice plans a direct-to-LDS configuration
# (9: 64x64, 7: 256x256, 8: 128x128, 10: 192x192 tiles).
WIDE_LDC = [((128, 8192, 2048), 9), ((256, 65536, 512), 7), ((768, 32768, 512), 8), ((192, 49152, 1024), 10)]


@pytest.mark.parametrize("shape,planned", WIDE_LDC, ids=[f"{m}x{n}x{k}-cfg{c}" for (m, n, k), c in WIDE_LDC])
def test_auto_plan_with_c_stride_past_32bit_offsets(sg, shape, planned):
    """The direct-to-LDS configurations address a tile of C with 32-bit
    offsets; with ldc so wide that 255 rows of C span more than 2 GiB the
    automatic call must switch to a register-staged kernel (64-bit
    addressing).  Integer inputs, checked bit for bit, with the columns past N
    left untouched."""
    M, N, K = shape
    ldc = 2_105_600
    assert (255 * ldc + 256) * 4 >= 1 << 31
    A, B, C0 = _inputs(M, N, K, "int4", 63 + planned)
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    st, _, cfg, _, _ = sg.sgemm_f32_ex_plan(0, 0, M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N)
    assert st == 0 and cfg == planned
    say(f"[wide_ldc] {shape} ldc={ldc} ({M * ldc * 4 / 2**30:.2f} GiB for C), planned configuration {cfg}")
    dC = torch.full((M, ldc), -7.25, device="cuda")
    dC[:, :N] = torch.from_numpy(C0).cuda()
    st = sg.sgemm_f32(M, N, K, 1.5, dA.data_ptr(), K, dB.data_ptr(), N, -0.5, dC.data_ptr(), ldc,
                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    C = dC[:, :N].cpu().numpy()
    assert np.all(dC[:, N:N + 256].cpu().numpy() == np.float32(-7.25))
    assert np.all(dC[:, -256:].cpu().numpy() == np.float32(-7.25))
    del dC
    torch.cuda.empty_cache()
    ok, info = check_full(C, A, B, 1.5, -0.5, C0, exact=True)
    assert ok, info


GRAPH_CASES = {"skinny": (16, 4096, 4096), "splitk": (512, 512, 8192), "kmajor": (4096, 16, 4096),
               "unaligned_split": (4096, 17, 4096), "packed": (2047, 2047, 2047)}


@pytest.mark.parametrize("case", sorted(GRAPH_CASES))
def test_split_plans_in_a_captured_graph(sg, case):
    """A call whose plan allocates stream-ordered scratch (the M <= 16 split,
    a tuned split-K plan, the N <= 16 streaming kernel's split, the 4-byte-load
    tiles with K split, operands copied to aligned rows), recorded into a
    graph: every replay, with eager work and synchronisation between replays,
    matches the eager result bit for bit."""
    M, N, K = GRAPH_CASES[case]
    say(f"[graph] {case} {M}x{N}x{K}")
    A, B, _ = _inputs(M, N, K, "uniform", 80, c0=False)
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    eager = torch.empty(M, N, device="cuda:0")
    out = torch.empty(M, N, device="cuda:0")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    assert sg.sgemm_f32(M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, eager.data_ptr(), N,
                        s.cuda_stream) == 0
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        st = sg.sgemm_f32(M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0, out.data_ptr(), N,
                          s.cuda_stream)
    assert st == 0
    want = eager.cpu().numpy()
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"replay {rep}"
        junk = torch.randn(1024, 1024, device="cuda:0") @ torch.randn(1024, 1024, device="cuda:0")
        torch.cuda.synchronize()
        del junk
    ok, info = check_full(want, A, B, 1.0, 0.0, None)
    assert ok, info
