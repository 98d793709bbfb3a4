"""GPU parity of every MFMA tile configuration, tile-row grouping and K split
that the tuning table can choose (sgemm_f32_ex_config), in all four operand
forms, against the oracle; and of the automatic plan on shapes whose class has
a tuned entry."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import check_full, from_device_padded, say, to_device_padded, zero_sum_integers

pytestmark = pytest.mark.gpu

FORMS = [(0, 0), (0, 1), (1, 0), (1, 1)]
FORM_IDS = ["nn", "nt", "tn", "tt"]


@pytest.fixture(scope="module")
def sg():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import fp32_sgemm_amd
    return fp32_sgemm_amd


def _stored(x, t):
    return np.ascontiguousarray(x.T) if t else x


def _inputs(M, N, K, dist, seed):
    w = workloads.custom(M, N, K, dist=dist, seed=seed, c0_dist="normal" if dist != "int4" else "int4")
    return workloads.make_inputs(w)


def run_cfg(sg, cfg, gm, splits, ta, tb, A, B, C0, alpha, beta, stream=None):
    M, K = A.shape
    N = B.shape[1]
    As, Bs = _stored(A, ta), _stored(B, tb)
    r4 = lambda x: (max(x, 1) + 3) // 4 * 4
    lda, ldb, ldc = r4(As.shape[1]), r4(Bs.shape[1]), N
    bA, pA, _ = to_device_padded(As, lda)
    bB, pB, _ = to_device_padded(Bs, ldb)
    bC, pC, _ = to_device_padded(C0, ldc, fill=np.float32(-7.25))
    s = stream or torch.cuda.current_stream()
    st = sg.sgemm_f32_ex_config(cfg, gm, splits, ta, tb, M, N, K, float(alpha), pA, lda, pB, ldb,
                                float(beta), pC, ldc, s.cuda_stream)
    torch.cuda.synchronize()
    return st, from_device_padded(bC, M, N, ldc), As, Bs


def check(C, As, Bs, ta, tb, alpha, beta, C0, exact):
    Cref, absab = oracle.sgemm_ref_op(As, Bs, ta, tb, alpha, beta, C0)
    if exact:
        return oracle.check_bitexact(C, Cref)
    return oracle.check_within_bound(C, Cref, oracle.error_bound(absab, alpha, beta, C0))


SHAPES = [(129, 127, 65), (300, 260, 700), (64, 64, 32), (257, 129, 1000), (130, 70, 9), (65, 200, 333)]
# Grid configurations (5, the persistent one, has tests of its own below).
GRID_CFGS = [0, 1, 2, 3, 4, 6]


@pytest.mark.parametrize("splits", [1, 2, 5])
@pytest.mark.parametrize("cfg", GRID_CFGS)
@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
def test_config_real(sg, cfg, splits, form, shape):
    M, N, K = shape
    ta, tb = form
    say(f"[cfg_real] cfg={cfg} splits={splits} {form} {shape}")
    A, B, C0 = _inputs(M, N, K, "uniform", 700 + M + N + K)
    st, C, As, Bs = run_cfg(sg, cfg, 8, splits, ta, tb, A, B, C0, 1.25, -0.5)
    assert st == 0
    ok, info = check(C, As, Bs, ta, tb, 1.25, -0.5, C0, exact=False)
    assert ok, info


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("cfg", GRID_CFGS)
@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
def test_config_integer_bitexact(sg, cfg, splits, form):
    """Integer-valued inputs are exact in FP32 in any summation order, so a
    split reduction must match bit for bit too."""
    M, N, K = 201, 157, 611
    ta, tb = form
    say(f"[cfg_int] cfg={cfg} splits={splits} {form}")
    A, B, C0 = _inputs(M, N, K, "int4", 800 + cfg)
    st, C, As, Bs = run_cfg(sg, cfg, 8, splits, ta, tb, A, B, C0, 2.0, -1.0)
    assert st == 0
    ok, info = check(C, As, Bs, ta, tb, 2.0, -1.0, C0, exact=True)
    assert ok, info


@pytest.mark.parametrize("gm", [1, 3, 16, 64])
@pytest.mark.parametrize("cfg", GRID_CFGS)
def test_tile_row_grouping(sg, cfg, gm):
    M, N, K = 1000, 900, 96
    say(f"[cfg_group] cfg={cfg} gm={gm}")
    A, B, C0 = _inputs(M, N, K, "int4", 900 + gm)
    st, C, As, Bs = run_cfg(sg, cfg, gm, 1, 0, 0, A, B, C0, 1.0, 1.0)
    assert st == 0
    ok, info = check(C, As, Bs, 0, 0, 1.0, 1.0, C0, exact=True)
    assert ok, info


def test_split_beta_zero_ignores_nan_c(sg):
    M, N, K = 130, 66, 400
    A, B, _ = _inputs(M, N, K, "uniform", 31)
    C0 = np.full((M, N), np.nan, np.float32)
    st, C, As, Bs = run_cfg(sg, 0, 8, 4, 0, 0, A, B, C0, 1.0, 0.0)
    assert st == 0 and np.all(np.isfinite(C))
    ok, info = check(C, As, Bs, 0, 0, 1.0, 0.0, None, exact=False)
    assert ok, info


def test_split_odd_n_scalar_reduction(sg):
    """N not a multiple of 4 takes the element-wise reduction."""
    M, N, K = 77, 63, 500
    A, B, C0 = _inputs(M, N, K, "uniform", 32)
    st, C, As, Bs = run_cfg(sg, 0, 8, 3, 0, 0, A, B, C0, 0.5, 2.0)
    assert st == 0
    ok, info = check(C, As, Bs, 0, 0, 0.5, 2.0, C0, exact=False)
    assert ok, info


def test_split_plans_on_two_streams(sg):
    """Two split products in flight on two streams: each stream's partials
    live in that call's own scratch."""
    M, N, K = 512, 512, 4096
    A1, B1, _ = _inputs(M, N, K, "uniform", 33)
    A2, B2, _ = _inputs(M, N, K, "uniform", 34)
    d = [torch.from_numpy(x).cuda() for x in (A1, B1, A2, B2)]
    C1 = torch.zeros(M, N, device="cuda:0")
    C2 = torch.zeros(M, N, device="cuda:0")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        assert sg.sgemm_f32_ex_config(0, 8, 4, 0, 0, M, N, K, 1.0, d[0].data_ptr(), K, d[1].data_ptr(), N,
                                      0.0, C1.data_ptr(), N, s1.cuda_stream) == 0
        assert sg.sgemm_f32_ex_config(2, 8, 8, 0, 0, M, N, K, 1.0, d[2].data_ptr(), K, d[3].data_ptr(), N,
                                      0.0, C2.data_ptr(), N, s2.cuda_stream) == 0
    torch.cuda.synchronize()
    for C, A, B in ((C1, A1, B1), (C2, A2, B2)):
        Cref, absab = oracle.sgemm_ref(A, B)
        ok, info = oracle.check_within_bound(C.cpu().numpy(), Cref, oracle.error_bound(absab, 1.0, 0.0, None))
        assert ok, info


def test_split_repeat_bitwise_identical(sg):
    M, N, K = 300, 400, 3000
    A, B, C0 = _inputs(M, N, K, "uniform", 35)
    r1 = run_cfg(sg, 3, 8, 6, 0, 1, A, B, C0, 1.0, 0.5)
    r2 = run_cfg(sg, 3, 8, 6, 0, 1, A, B, C0, 1.0, 0.5)
    assert r1[0] == 0 and r2[0] == 0
    assert np.array_equal(r1[1].view(np.uint32), r2[1].view(np.uint32))


TUNED_SHAPES = [(1024, 1024, 1024), (2048, 2048, 2048), (512, 512, 8192), (4096, 1024, 256),
                (256, 4096, 4096), (2048, 2048, 512), (3000, 3000, 3000), (5000, 3000, 200),
                (1536, 1536, 4096), (1600, 1600, 4096), (6144, 3072, 1024)]


@pytest.mark.parametrize("shape", TUNED_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in TUNED_SHAPES])
def test_automatic_plan(sg, shape):
    """sgemm_f32 on shapes across the table's classes, whatever plan the table
    gives, checked element by element."""
    M, N, K = shape
    A, B, C0 = _inputs(M, N, K, "uniform", 36 + M // 64)
    st_p = sg.sgemm_f32_ex_plan(0, 0, M, N, K, 1.5, 0x100000, K, 0x100000, N)
    say(f"[auto_plan] {shape} plan={st_p}")
    dA, dB, dC = (torch.from_numpy(x).cuda() for x in (A, B, C0))
    st = sg.sgemm_f32(M, N, K, 1.5, dA.data_ptr(), K, dB.data_ptr(), N, -0.5, dC.data_ptr(), N,
                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    C = dC.cpu().numpy()
    ok, info = check_full(C, A, B, 1.5, -0.5, C0)
    assert ok, info


# ---------------------------------------------------------------------------
# Persistent stream-K configuration (5): whole-tile rounds, then K-slice
# shares; shapes with fewer tiles than resident work-groups (most work-groups
# idle, tiles shared by several), with whole rounds plus a remainder, and with
# a K tail inside shared tiles.
# ---------------------------------------------------------------------------
SK_SMALL = [(129, 127, 65), (300, 260, 700), (64, 64, 32), (1000, 900, 96), (257, 4000, 1000),
            (640, 640, 4099)]
SK_LARGE = [(3000, 3000, 700), (4092, 2900, 333), (2900, 4100, 64)]


@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("shape", SK_SMALL, ids=[f"{m}x{n}x{k}" for m, n, k in SK_SMALL])
def test_streamk_real(sg, form, shape):
    M, N, K = shape
    ta, tb = form
    say(f"[streamk_real] {form} {shape}")
    A, B, C0 = _inputs(M, N, K, "uniform", 1100 + M + N + K)
    st, C, As, Bs = run_cfg(sg, 5, 8, 1, ta, tb, A, B, C0, 1.25, -0.5)
    assert st == 0
    ok, info = check(C, As, Bs, ta, tb, 1.25, -0.5, C0, exact=False)
    assert ok, info


@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("shape", SK_SMALL + SK_LARGE, ids=[f"{m}x{n}x{k}" for m, n, k in SK_SMALL + SK_LARGE])
def test_streamk_integer_bitexact(sg, form, shape):
    M, N, K = shape
    ta, tb = form
    say(f"[streamk_int] {form} {shape}")
    A, B, C0 = _inputs(M, N, K, "int4", 1200 + M + N + K)
    st, C, As, Bs = run_cfg(sg, 5, 8, 1, ta, tb, A, B, C0, 1.0, 2.0)
    assert st == 0
    ok, info = check(C, As, Bs, ta, tb, 1.0, 2.0, C0, exact=True)
    assert ok, info


@pytest.mark.parametrize("shape", SK_LARGE, ids=[f"{m}x{n}x{k}" for m, n, k in SK_LARGE])
def test_streamk_real_large(sg, shape):
    M, N, K = shape
    say(f"[streamk_real_large] {shape}")
    A, B, C0 = _inputs(M, N, K, "uniform", 1300 + M + N + K)
    st, C, As, Bs = run_cfg(sg, 5, 8, 1, 0, 0, A, B, C0, 1.5, -0.5)
    assert st == 0
    ok, info = check_full(C, A, B, 1.5, -0.5, C0)
    assert ok, info


def test_streamk_wide_workload(sg):
    """The 4096 x 11008 x 512 workload (2752 tiles: five whole rounds and a
    partial one on 512 resident work-groups) through the persistent kernel."""
    w = workloads.WORKLOADS["wide4096x11008x512"]
    say("[streamk_wide]")
    A, B, C0 = workloads.make_inputs(w)
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    dC = torch.full((w.M, w.N), float("nan"), device="cuda:0")
    st = sg.sgemm_f32_ex_config(5, 8, 1, 0, 0, w.M, w.N, w.K, w.alpha, dA.data_ptr(), w.K, dB.data_ptr(), w.N,
                                w.beta, dC.data_ptr(), w.N, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    C = dC.cpu().numpy()
    assert np.all(np.isfinite(C))
    ok, info = check_full(C, A, B, w.alpha, w.beta, C0)
    assert ok, info


def test_streamk_repeat_bitwise_identical(sg):
    M, N, K = 3000, 3000, 700
    A, B, C0 = _inputs(M, N, K, "uniform", 37)
    r1 = run_cfg(sg, 5, 8, 1, 0, 0, A, B, C0, 1.0, 0.5)
    r2 = run_cfg(sg, 5, 8, 1, 0, 0, A, B, C0, 1.0, 0.5)
    assert r1[0] == 0 and r2[0] == 0
    assert np.array_equal(r1[1].view(np.uint32), r2[1].view(np.uint32))


# ---------------------------------------------------------------------------
# Configurations 7, 8, 9 and 10: the kernel that copies the operands straight
# into LDS, on 256x256, 128x128, 64x64 and 192x192 tiles.  M, N and K multiples of 4;
# edge tiles get zeros past M, N and K in LDS and masked stores.  One slice is
# 16 deep and three are fetched ahead, so short K exercises the repeated loads
# past the end.
# ---------------------------------------------------------------------------
BIG_CFGS = [7, 8, 9, 10]

# Extents that are not multiples of 4 on operands stored along k (M of A as
# given, N of B given transposed): (form, M, N, K).  Rows past the edge read
# as zeros; the other extents stay multiples of 4.
ODD_KROWS = [((0, 0), 257, 512, 64), ((0, 1), 131, 133, 36), ((0, 0), 511, 260, 1028), ((0, 1), 258, 515, 48),
             ((1, 1), 256, 515, 20), ((0, 0), 1, 388, 16), ((1, 1), 200, 3, 100)]


@pytest.mark.parametrize("cfg", BIG_CFGS)
@pytest.mark.parametrize("case", ODD_KROWS, ids=[f"{FORM_IDS[2 * f[0] + f[1]]}-{m}x{n}x{k}" for f, m, n, k in ODD_KROWS])
def test_big_configs_odd_extents_along_k(sg, cfg, case):
    (ta, tb), M, N, K = case
    say(f"[big_odd] cfg {cfg} {case}")
    A, B, C0 = _inputs(M, N, K, "uniform", 40 + M + N)
    st, C, As, Bs = run_cfg(sg, cfg, 8, 1, ta, tb, A, B, C0, 1.5, -0.5)
    assert st == 0
    ok, info = check(C, As, Bs, ta, tb, 1.5, -0.5, C0, exact=False)
    assert ok, info
    Ai, Bi, Ci = _inputs(M, N, K, "int4", 50 + M + N)
    st, C, As, Bs = run_cfg(sg, cfg, 8, 1, ta, tb, Ai, Bi, Ci, -1.0, 1.0)
    assert st == 0
    ok, info = check(C, As, Bs, ta, tb, -1.0, 1.0, Ci, exact=True)
    assert ok, info

BIG_SHAPES = [(256, 512, 16), (512, 256, 48), (768, 512, 272), (512, 768, 1024), (128, 384, 32),
              (64, 192, 64),
              # edge tiles: M, N not multiples of the tile, K not of 16 (multiples of 4)
              (260, 516, 20), (252, 256, 36), (516, 260, 100), (4, 8, 4), (132, 388, 52), (124, 132, 16),
              (68, 60, 28),
              # 192x192 tiles: whole, and edges of 4 to 188
              (384, 576, 48), (196, 388, 20), (580, 200, 116),
              # K >= 2048 on a grid of at most one tile per CU: two groups of
              # waves per 128x128 tile (and per 64x64 tile)
              (384, 640, 2068)]


@pytest.mark.parametrize("cfg", BIG_CFGS)
@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("shape", BIG_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in BIG_SHAPES])
def test_big_kernel_real(sg, cfg, form, shape):
    M, N, K = shape
    ta, tb = form
    say(f"[big_real] cfg {cfg} {form} {shape}")
    A, B, C0 = _inputs(M, N, K, "uniform", 900 + M + N + K)
    st, C, As, Bs = run_cfg(sg, cfg, 8, 1, ta, tb, A, B, C0, 1.25, -0.5)
    assert st == 0
    ok, info = check(C, As, Bs, ta, tb, 1.25, -0.5, C0, exact=False)
    assert ok, info


@pytest.mark.parametrize("cfg", BIG_CFGS)
@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
def test_big_kernel_integer_bitexact(sg, cfg, form):
    M, N, K = 516, 772, 404
    ta, tb = form
    say(f"[big_int] cfg {cfg} {form}")
    A, B, C0 = _inputs(M, N, K, "int4", 910)
    st, C, As, Bs = run_cfg(sg, cfg, 8, 1, ta, tb, A, B, C0, 1.5, -0.5)
    assert st == 0
    ok, info = check(C, As, Bs, ta, tb, 1.5, -0.5, C0, exact=True)
    assert ok, info


@pytest.mark.parametrize("cfg", BIG_CFGS)
def test_big_kernel_beta_zero_ignores_nan_c(sg, cfg):
    M, N, K = 512, 512, 64
    A, B, _ = _inputs(M, N, K, "uniform", 911)
    C0 = np.full((M, N), np.nan, np.float32)
    st, C, As, Bs = run_cfg(sg, cfg, 8, 1, 0, 0, A, B, C0, 1.0, 0.0)
    assert st == 0 and np.all(np.isfinite(C))
    ok, info = check(C, As, Bs, 0, 0, 1.0, 0.0, None, exact=False)
    assert ok, info


@pytest.mark.parametrize("cfg", [8, 9, 10])
def test_direct_lds_grouping_bitwise(sg, cfg):
    """The grouping changes only the order of the tiles: every grouping gives
    the same bits."""
    M, N, K = 1024, 640, 160
    A, B, C0 = _inputs(M, N, K, "uniform", 915)
    ref = None
    for gm in (1, 3, 8, 64):
        st, C, _, _ = run_cfg(sg, cfg, gm, 1, 0, 0, A, B, C0, 1.0, 0.5)
        assert st == 0
        if ref is None:
            ref = C
        assert np.array_equal(C.view(np.uint32), ref.view(np.uint32)), gm


@pytest.mark.parametrize("cfg", BIG_CFGS)
@pytest.mark.parametrize("form", [(0, 0), (1, 1)], ids=["nn", "tt"])
def test_big_kernel_padded_strides(sg, cfg, form):
    """Row strides wider than the stored rows (multiples of 4), C included."""
    M, N, K = 512, 512, 96
    ta, tb = form
    A, B, C0 = _inputs(M, N, K, "uniform", 912)
    As, Bs = _stored(A, ta), _stored(B, tb)
    lda, ldb, ldc = As.shape[1] + 12, Bs.shape[1] + 4, N + 20
    bA, pA, _ = to_device_padded(As, lda)
    bB, pB, _ = to_device_padded(Bs, ldb)
    bC, pC, _ = to_device_padded(C0, ldc, fill=np.float32(-7.25))
    st = sg.sgemm_f32_ex_config(cfg, 8, 1, ta, tb, M, N, K, 0.75, pA, lda, pB, ldb, 0.5, pC, ldc,
                                torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    host = bC.cpu().numpy()
    C = from_device_padded(bC, M, N, ldc)
    ok, info = check(C, As, Bs, ta, tb, 0.75, 0.5, C0, exact=False)
    assert ok, info
    # the padding between rows of C is untouched
    gaps = np.lib.stride_tricks.as_strided(host[N:], shape=(M - 1, ldc - N), strides=(ldc * 4, 4))
    assert np.all(gaps == np.float32(-7.25))


@pytest.mark.parametrize("cfg", BIG_CFGS)
def test_big_kernel_rejects_what_it_cannot_cover(sg, cfg):
    """K, or the extent of an operand stored along M or N (N of B as given,
    M of A given transposed), not a multiple of 4: refused before any launch."""
    for (ta, tb), (M, N, K) in (((0, 0), (256, 258, 64)), ((1, 1), (258, 256, 64)), ((0, 1), (256, 256, 66))):
        A, B, C0 = _inputs(M, N, K, "uniform", 913)
        st, _, _, _ = run_cfg(sg, cfg, 8, 1, ta, tb, A, B, C0, 1.0, 0.0)
        assert st == sg.ERR_NOT_APPLICABLE, (ta, tb, M, N, K)


@pytest.mark.parametrize("cfg", BIG_CFGS)
@pytest.mark.parametrize("K", [65536, 65540])
def test_big_kernel_long_k_bitexact(sg, cfg, K):
    """4096 slices through the four LDS stages (and a K tail of 4): integer
    inputs keep every partial sum below 2**24, so the result is exact."""
    M, N = 256, 512
    say(f"[big_long_k] cfg {cfg} K={K}")
    A, B, C0 = _inputs(M, N, K, "int4", 914 + K % 16)
    st, C, As, Bs = run_cfg(sg, cfg, 8, 1, 0, 0, A, B, C0, 1.0, -1.0)
    assert st == 0
    ok, info = check(C, As, Bs, 0, 0, 1.0, -1.0, C0, exact=True)
    assert ok, info


ALL_CFGS = [(c, 1) for c in range(11)] + [(c, 3) for c in GRID_CFGS]


@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("cfg_splits", ALL_CFGS, ids=[f"cfg{c}_s{s}" for c, s in ALL_CFGS])
def test_negative_alpha_zero_sums_bitexact(sg, cfg_splits, form):
    """alpha < 0 with beta = 0 writes alpha * acc without adding anything: an
    exactly zero sum is -0 (the oracle's IEEE value), in every plan, split or
    not; the rest of the integer-valued product is exact."""
    cfg, splits = cfg_splits
    ta, tb = form
    M, N, K = 260, 132, 196
    say(f"[neg_alpha_zero] cfg={cfg} splits={splits} {form}")
    A, B = zero_sum_integers(M, N, K, 71 + cfg)
    C0 = np.full((M, N), np.nan, np.float32)
    st, C, As, Bs = run_cfg(sg, cfg, 8, splits, ta, tb, A, B, C0, -2.0, 0.0)
    assert st == 0
    assert np.all(np.signbit(C[1, :])) and np.all(C[1, :] == 0)
    ok, info = check(C, As, Bs, ta, tb, -2.0, 0.0, None, exact=True)
    assert ok, info
