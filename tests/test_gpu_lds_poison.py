"""The LDS-poisoning debug copy of the library (built with SGEMM_LDS_POISON):
every kernel fills its LDS with quiet NaNs before its first load.  A stage read
before the loads that fill it have landed (for the kernels that copy operands
straight into LDS and order their stages with vector-memory counts and a bare
s_barrier), or a part of LDS that is read but never written, would turn entries
of C into NaN.  On integer-valued inputs the result is exact, so every case is
compared bit for bit with the oracle: short K (slices loaded past the end),
edge tiles, long K (thousands of slices through the stages), all four operand
forms, every tile configuration, the VALU kernel, the streaming kernels for
M <= 32 (plain form) and M or N <= 16 (rows along k), and both 16-bit kernels.  Calls go through the debug library's C interface."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import from_device_padded, say, to_device_padded

pytestmark = pytest.mark.gpu

FORMS = [(0, 0), (0, 1), (1, 0), (1, 1)]
FORM_IDS = ["nn", "nt", "tn", "tt"]


@pytest.fixture(scope="module")
def plib():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import fp32_sgemm_amd
    return fp32_sgemm_amd.lds_poison_library()


def _stored(x, t):
    return np.ascontiguousarray(x.T) if t else x


def _int_inputs(M, N, K, seed):
    w = workloads.custom(M, N, K, dist="int4", seed=seed, c0_dist="int4")
    return workloads.make_inputs(w)


def _run_config(plib, cfg, gm, splits, ta, tb, A, B, C0, alpha, beta):
    M, K = A.shape
    N = B.shape[1]
    As, Bs = _stored(A, ta), _stored(B, tb)
    r4 = lambda x: (max(x, 1) + 3) // 4 * 4
    lda, ldb, ldc = r4(As.shape[1]), r4(Bs.shape[1]), N
    bA, pA, _ = to_device_padded(As, lda)
    bB, pB, _ = to_device_padded(Bs, ldb)
    bC, pC, _ = to_device_padded(C0, ldc, fill=np.float32(-7.25))
    st = plib.sgemm_f32_ex_config(cfg, gm, splits, ta, tb, M, N, K, ctypes.c_float(alpha), pA, lda, pB, ldb,
                                  ctypes.c_float(beta), pC, ldc, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return st, from_device_padded(bC, M, N, ldc)


def _exact(C, A, B, alpha, beta, C0):
    assert not np.any(np.isnan(C)), "NaN in C: an LDS stage was read before it was filled"
    Cref, _ = oracle.sgemm_ref(A, B, alpha, beta, C0)
    return oracle.check_bitexact(C, Cref)


BIG_SHAPES = [(256, 512, 16), (512, 256, 48), (768, 512, 272), (512, 768, 1024), (128, 384, 32),
              (64, 192, 64), (260, 516, 20), (252, 256, 36), (516, 260, 100), (4, 8, 4), (132, 388, 52),
              (124, 132, 16), (68, 60, 28), (384, 576, 48), (196, 388, 20)]


@pytest.mark.parametrize("cfg", [7, 8, 9, 10])
@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("shape", BIG_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in BIG_SHAPES])
def test_poisoned_direct_lds_kernel(plib, cfg, form, shape):
    M, N, K = shape
    ta, tb = form
    say(f"[poison_big] cfg {cfg} {form} {shape}")
    A, B, C0 = _int_inputs(M, N, K, 1500 + M + N + K)
    st, C = _run_config(plib, cfg, 8, 1, ta, tb, A, B, C0, 1.5, -0.5)
    assert st == 0
    ok, info = _exact(C, A, B, 1.5, -0.5, C0)
    assert ok, info


# Extents that are not multiples of 4 on operands stored along k: (form, M, N, K).
ODD_KROWS = [((0, 0), 257, 512, 64), ((0, 1), 131, 133, 36), ((1, 1), 256, 515, 20), ((0, 0), 511, 260, 1028)]


@pytest.mark.parametrize("cfg", [7, 8, 9, 10])
@pytest.mark.parametrize("case", ODD_KROWS, ids=[f"{FORM_IDS[2 * f[0] + f[1]]}-{m}x{n}x{k}" for f, m, n, k in ODD_KROWS])
def test_poisoned_direct_lds_kernel_odd_extents(plib, cfg, case):
    (ta, tb), M, N, K = case
    say(f"[poison_big_odd] cfg {cfg} {case}")
    A, B, C0 = _int_inputs(M, N, K, 1550 + M + N)
    st, C = _run_config(plib, cfg, 8, 1, ta, tb, A, B, C0, 1.5, -0.5)
    assert st == 0
    ok, info = _exact(C, A, B, 1.5, -0.5, C0)
    assert ok, info


@pytest.mark.parametrize("cfg", [7, 8, 9, 10])
@pytest.mark.parametrize("K", [65536, 65540])
def test_poisoned_direct_lds_kernel_long_k(plib, cfg, K):
    M, N = 256, 512
    say(f"[poison_long_k] cfg {cfg} K={K}")
    A, B, C0 = _int_inputs(M, N, K, 1600 + K % 16)
    st, C = _run_config(plib, cfg, 8, 1, 0, 0, A, B, C0, 1.0, -1.0)
    assert st == 0
    ok, info = _exact(C, A, B, 1.0, -1.0, C0)
    assert ok, info


REG_SHAPES = [(129, 127, 65), (300, 260, 700), (64, 64, 32), (130, 70, 9)]


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("shape", REG_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in REG_SHAPES])
def test_poisoned_register_staged_kernels(plib, cfg, splits, shape):
    if cfg == 5 and splits > 1:
        pytest.skip("the stream-K configuration takes no split count")
    M, N, K = shape
    say(f"[poison_reg] cfg {cfg} splits {splits} {shape}")
    A, B, C0 = _int_inputs(M, N, K, 1700 + cfg)
    for ta, tb in ((0, 0), (1, 1)):
        st, C = _run_config(plib, cfg, 8, splits, ta, tb, A, B, C0, 2.0, -1.0)
        assert st == 0
        ok, info = _exact(C, A, B, 2.0, -1.0, C0)
        assert ok, (ta, tb, info)


@pytest.mark.parametrize("variant,M,N", [(3, 300, 1000), (4, 16, 1000), (4, 24, 1000), (4, 20, 4200)],
                         ids=["valu", "skinny16", "skinny24", "skinny20_wide"])   # the VALU kernel, the M <= 32 kernel
def test_poisoned_valu_and_skinny(plib, variant, M, N):
    K = 3000
    say(f"[poison_variant] {variant} M={M} N={N}")
    A, B, C0 = _int_inputs(M, N, K, 1800 + variant)
    dA, dB, dC = (torch.from_numpy(x).cuda() for x in (A, B, C0))
    st = plib.sgemm_f32_variant(variant, M, N, K, ctypes.c_float(1.0), dA.data_ptr(), K, dB.data_ptr(), N,
                                ctypes.c_float(1.0), dC.data_ptr(), N, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    ok, info = _exact(dC.cpu().numpy(), A, B, 1.0, 1.0, C0)
    assert ok, info


@pytest.mark.parametrize("case", [(0, 1, 16, 1000, 3000), (1, 1, 13, 1000, 3000), (0, 0, 1000, 16, 3000),
                                  (0, 1, 4, 16384, 2000), (0, 1, 16, 4096, 2048), (0, 1, 4096, 13, 2000)],
                         ids=["nt", "tt", "nn_tall", "nt_long_k", "nt_staged", "nt_tall_staged"])
def test_poisoned_skinny_kmajor(plib, case):
    """The streaming kernel for operands whose rows run along k (B given
    N x K with M <= 16, A as given with N <= 16)."""
    ta, tb, M, N, K = case
    say(f"[poison_kmaj] {case}")
    A, B, C0 = _int_inputs(M, N, K, 1850 + M + N)
    As, Bs = _stored(A, ta), _stored(B, tb)
    dA, dB, dC = (torch.from_numpy(x).cuda() for x in (As, Bs, C0))
    st = plib.sgemm_f32_ex_variant(4, ta, tb, M, N, K, ctypes.c_float(1.0), dA.data_ptr(), As.shape[1],
                                   dB.data_ptr(), Bs.shape[1], ctypes.c_float(1.0), dC.data_ptr(), N,
                                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    ok, info = _exact(dC.cpu().numpy(), A, B, 1.0, 1.0, C0)
    assert ok, info


# 16-bit inputs: (M, N, K); 4096 x 4096 runs the larger-tile kernel (at least
# 256 tiles of 256 x 256), the others the 128 x 128 kernel.
G16_SHAPES = [(4096, 4096, 8), (4096, 4096, 192), (4096, 4096, 520), (4096, 3904, 576), (300, 260, 700),
              (128, 128, 64), (1000, 1000, 576), (2048, 1040, 192), (3000, 2904, 192), (16, 2048, 2048)]


@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("kind", [1, 2], ids=["bf16", "f16"])
@pytest.mark.parametrize("shape", G16_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in G16_SHAPES])
def test_poisoned_16bit_kernels(plib, kind, shape, form):
    """All four operand forms: A transposed (K x M) and B as given (K x N)
    are read in place with transposing LDS reads by the direct-to-LDS kernel
    when K is a multiple of 64, packed otherwise; 256 x 256 tiles on the
    4096-wide grids, 192 x 192 on 3000 x 2904, 128 x 128 tiles (two
    work-groups per CU) on the others, with edge tiles and one to nine
    slices; 16 x 2048 x 2048 splits K over 8 work-groups per tile."""
    M, N, K = shape
    ta, tb = form
    say(f"[poison_16] kind {kind} {shape} form={form}")
    w = workloads.custom(M, N, K, dist="int4", seed=1900 + K, c0_dist="int4")
    A16, B16, C0 = workloads.make_inputs_16bit(w, kind)
    As = np.ascontiguousarray(A16.T) if ta else A16
    Bs = np.ascontiguousarray(B16.T) if tb else B16
    dA = torch.from_numpy(As.view(np.int16)).cuda()
    dB = torch.from_numpy(Bs.view(np.int16)).cuda()
    dC = torch.from_numpy(C0).cuda()
    st = plib.gemm16_f32(kind, ta, tb, M, N, K, ctypes.c_float(1.0), dA.data_ptr(), As.shape[1], dB.data_ptr(),
                         Bs.shape[1], ctypes.c_float(-1.0), dC.data_ptr(), N, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    C = dC.cpu().numpy()
    assert not np.any(np.isnan(C)), "NaN in C: an LDS stage was read before it was filled"
    Cref, _ = oracle.sgemm_ref(oracle.decode_16(A16, kind), oracle.decode_16(B16, kind), 1.0, -1.0, C0)
    ok, info = oracle.check_bitexact(C, Cref)
    assert ok, info
