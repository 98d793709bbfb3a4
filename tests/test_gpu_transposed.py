"""GPU parity for transposed operands: sgemm_f32_ex / sgemm_f32_ex_variant
against the oracle's transposed-operand form.

C = alpha*op(A)*op(B) + beta*C0, where a transposed operand is stored as the
transpose of its op() (A as K x M, B as N x K) and the library reads it in that
layout.  The same bars as for the plain form: real-valued inputs within
2e-5 * (|alpha|*(|op(A)||op(B)|)_ij + |beta|*|C0_ij|) per element, integer-valued
inputs bit for bit; full-size products element by element against the oracle
evaluated on op(A) and op(B) themselves.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import check_full, from_device_padded, say, to_device_padded

pytestmark = pytest.mark.gpu

FORMS = [(0, 0), (0, 1), (1, 0), (1, 1)]
FORM_IDS = ["nn", "nt", "tn", "tt"]
VID = {"auto": 0, "mfma_large": 1, "mfma_small": 2, "valu": 3, "skinny": 4, "mfma_scalar": 5}
VECTOR_ONLY = (1, 2)


@pytest.fixture(scope="module")
def sg():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import fp32_sgemm_amd
    return fp32_sgemm_amd


def _stored(x, trans):
    return np.ascontiguousarray(x.T) if trans else x


def run_ex(sg, variant, ta, tb, A, B, C0, alpha, beta, lda=None, ldb=None, ldc=None,
           offs=(0, 0, 0), c_fill=np.nan):
    """A (M x K) and B (K x N) are op(A) and op(B); they are stored transposed
    when the flag says so.  Returns (status, C, stored A, stored B)."""
    M, K = A.shape
    N = B.shape[1]
    As, Bs = _stored(A, ta), _stored(B, tb)
    r4 = (lambda x: (max(x, 1) + 3) // 4 * 4) if variant in VECTOR_ONLY else (lambda x: max(x, 1))
    lda = lda or r4(As.shape[1])
    ldb = ldb or r4(Bs.shape[1])
    ldc = ldc or max(N, 1)
    bA, pA, _ = to_device_padded(As, lda, offs[0])
    bB, pB, _ = to_device_padded(Bs, ldb, offs[1])
    Cinit = C0 if C0 is not None else np.full((M, N), c_fill, np.float32)
    bC, pC, _ = to_device_padded(Cinit, ldc, offs[2], fill=np.float32(-7.25))
    s = torch.cuda.current_stream()
    st = sg.sgemm_f32_ex_variant(variant, ta, tb, M, N, K, float(alpha), pA, lda, pB, ldb,
                                 float(beta), pC, ldc, s.cuda_stream)
    torch.cuda.synchronize()
    C = from_device_padded(bC, M, N, ldc, offs[2])
    return st, C, As, Bs


def check_op_full(C, As, Bs, ta, tb, alpha, beta, C0, exact=False):
    Cref, absab = oracle.sgemm_ref_op(As, Bs, ta, tb, alpha, beta, C0)
    if exact:
        return oracle.check_bitexact(C, Cref)
    return oracle.check_within_bound(C, Cref, oracle.error_bound(absab, alpha, beta, C0))


def _inputs(M, N, K, dist, seed, c0=True):
    w = workloads.custom(M, N, K, dist=dist, seed=seed,
                         c0_dist=("normal" if dist != "int4" else "int4") if c0 else None)
    return workloads.make_inputs(w)


RAGGED = [(1, 1, 1), (2, 3, 5), (17, 31, 33), (63, 65, 127), (129, 127, 65),
          (300, 260, 70), (257, 129, 1000), (128, 128, 128), (96, 200, 31), (130, 70, 9),
          (16, 300, 200), (5, 7, 300)]
MFMA = ["auto", "mfma_large", "mfma_small", "mfma_scalar"]


@pytest.mark.parametrize("variant", MFMA)
@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("shape", RAGGED, ids=[f"{m}x{n}x{k}" for m, n, k in RAGGED])
def test_ragged_real(sg, variant, form, shape):
    M, N, K = shape
    ta, tb = form
    say(f"[t_ragged_real] {variant} {form} {shape}")
    A, B, C0 = _inputs(M, N, K, "uniform", 500 + M + N + K)
    st, C, As, Bs = run_ex(sg, VID[variant], ta, tb, A, B, C0, 1.25, -0.5)
    assert st == 0
    ok, info = check_op_full(C, As, Bs, ta, tb, 1.25, -0.5, C0)
    assert ok, info


@pytest.mark.parametrize("variant", MFMA)
@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("shape", RAGGED, ids=[f"{m}x{n}x{k}" for m, n, k in RAGGED])
def test_ragged_integer_bitexact(sg, variant, form, shape):
    M, N, K = shape
    ta, tb = form
    say(f"[t_ragged_int] {variant} {form} {shape}")
    A, B, C0 = _inputs(M, N, K, "int4", 600 + M + N + K)
    st, C, As, Bs = run_ex(sg, VID[variant], ta, tb, A, B, C0, 1.5, -0.5)
    assert st == 0
    ok, info = check_op_full(C, As, Bs, ta, tb, 1.5, -0.5, C0, exact=True)
    assert ok, info


@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("variant", ["auto", "mfma_scalar"])
def test_odd_strides_and_misaligned(sg, form, variant):
    ta, tb = form
    M, N, K = 141, 97, 61
    A, B, C0 = _inputs(M, N, K, "uniform", 19)
    wa = M if ta else K
    wb = K if tb else N
    st, C, As, Bs = run_ex(sg, VID[variant], ta, tb, A, B, C0, 0.5, 0.25, lda=wa + 1, ldb=wb + 3,
                           ldc=N + 2, offs=(1, 3, 1))
    assert st == 0
    ok, info = check_op_full(C, As, Bs, ta, tb, 0.5, 0.25, C0)
    assert ok, info


@pytest.mark.parametrize("form", FORMS[1:], ids=FORM_IDS[1:])
def test_unaligned_operands_packed(sg, form):
    """Odd row strides of transposed operands on a larger product: copied
    into aligned scratch rows first."""
    ta, tb = form
    M, N, K = 1700, 1500, 1600
    A, B, C0 = _inputs(M, N, K, "uniform", 26)
    wa = M if ta else K
    wb = K if tb else N
    say(f"[t_packed] {form}")
    st, C, As, Bs = run_ex(sg, VID["auto"], ta, tb, A, B, C0, 0.75, 0.5, lda=wa + 1, ldb=wb + 1)
    assert st == 0
    assert sg.sgemm_f32_ex_plan(ta, tb, M, N, K, 1.0, 256, wa + 1, 256, wb + 1)[1] != sg.MFMA_SCALAR
    ok, info = check_op_full(C, As, Bs, ta, tb, 0.75, 0.5, C0)
    assert ok, info


def test_transposed_a_straddling_edge_split(sg):
    """A stored K x M with M not a multiple of 4 (its 16-byte groups straddle
    the M edge): the automatic plan splits K."""
    M, N, K = 2047, 512, 4096
    say("[t_straddle] tn 2047x512x4096")
    assert sg.sgemm_f32_ex_plan(1, 0, M, N, K, 1.0, 256, 2048, 256, N)[4] > 1
    A, B, C0 = _inputs(M, N, K, "uniform", 27)
    st, C, As, Bs = run_ex(sg, VID["auto"], 1, 0, A, B, C0, 0.75, 0.5, lda=2048)
    assert st == 0
    ok, info = check_op_full(C, As, Bs, 1, 0, 0.75, 0.5, C0)
    assert ok, info


@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
def test_beta_zero_ignores_nan_c(sg, form):
    ta, tb = form
    A, B, _ = _inputs(150, 140, 90, "uniform", 20, c0=False)
    st, C, As, Bs = run_ex(sg, 0, ta, tb, A, B, None, 1.0, 0.0, c_fill=np.nan)
    assert st == 0 and np.all(np.isfinite(C))
    ok, info = check_op_full(C, As, Bs, ta, tb, 1.0, 0.0, None)
    assert ok, info


def test_skinny_kmajor_refuses_more_than_16_rows(sg):
    for ta, tb, M, N in ((0, 1, 17, 64), (1, 1, 17, 64), (0, 0, 64, 17), (0, 1, 64, 17)):
        A, B, C0 = _inputs(M, N, 64, "uniform", 25)
        st, _, _, _ = run_ex(sg, VID["skinny"], ta, tb, A, B, C0, 1.0, 0.0)
        assert st == sg.ERR_NOT_APPLICABLE, (ta, tb, M, N)


@pytest.mark.parametrize("form", FORMS[1:], ids=FORM_IDS[1:])
def test_unsupported_variants_refuse(sg, form):
    ta, tb = form
    A, B, C0 = _inputs(16, 64, 64, "uniform", 21)
    st, _, _, _ = run_ex(sg, VID["valu"], ta, tb, A, B, C0, 1.0, 0.0)
    assert st == sg.ERR_NOT_APPLICABLE
    if form == (1, 0):   # A transposed with B as given: no streaming form
        st, _, _, _ = run_ex(sg, VID["skinny"], ta, tb, A, B, C0, 1.0, 0.0)
        assert st == sg.ERR_NOT_APPLICABLE


# The streaming kernel on operands whose rows run along k: B given N x K with
# M <= 16 (NT, TT), and A as given with N <= 16 (NN, NT; C written
# transposed).  (ta, tb, M, N, K): ragged row counts of the streamed side
# (edge work-groups of 32 rows), K tails inside a 64-deep batch, splits of K
# over work-groups with 0 to 8 batches per wave (two or three in flight).
SKINNY_KMAJ = [(0, 1, 16, 4096, 300), (0, 1, 1, 1, 1), (0, 1, 3, 33, 100), (0, 1, 16, 2050, 1000),
               (0, 1, 13, 4093, 777), (0, 1, 16, 100, 4099), (0, 1, 15, 16, 17), (0, 1, 16, 200, 8191),
               (1, 1, 16, 4096, 300), (1, 1, 5, 130, 777), (1, 1, 16, 257, 513), (1, 1, 1, 4097, 65),
               (0, 0, 4096, 16, 300), (0, 0, 1000, 1, 77), (0, 0, 2050, 16, 1000), (0, 0, 33, 11, 4099),
               (0, 0, 4093, 14, 777), (0, 0, 100, 3, 8191), (0, 1, 4096, 16, 300), (0, 1, 130, 9, 2000),
               (0, 1, 2051, 16, 64), (0, 1, 4, 16384, 2000), (0, 0, 16384, 8, 1280), (1, 1, 12, 16000, 700),
               (0, 0, 4096, 1, 300), (0, 0, 16400, 5, 1700),
               # X read along k staged in LDS (splits of 512 to 1024 k)
               (0, 1, 16, 4096, 4096), (0, 1, 13, 4093, 2000), (0, 1, 4093, 11, 3000)]
KMAJ_IDS = [f"{FORM_IDS[2 * ta + tb]}-{m}x{n}x{k}" for ta, tb, m, n, k in SKINNY_KMAJ]


@pytest.mark.parametrize("variant", ["skinny", "auto"])
@pytest.mark.parametrize("case", SKINNY_KMAJ, ids=KMAJ_IDS)
def test_skinny_kmajor_forms(sg, variant, case):
    ta, tb, M, N, K = case
    say(f"[t_skinny_kmaj] {variant} {case}")
    A, B, C0 = _inputs(M, N, K, "uniform", 700 + M + N + K)
    st, C, As, Bs = run_ex(sg, VID[variant], ta, tb, A, B, C0, -0.75, 2.0)
    assert st == 0
    ok, info = check_op_full(C, As, Bs, ta, tb, -0.75, 2.0, C0)
    assert ok, info
    Ai, Bi, _ = _inputs(M, N, K, "int4", 800 + M + N + K, c0=False)
    st, C, As, Bs = run_ex(sg, VID[variant], ta, tb, Ai, Bi, None, 1.0, 0.0)
    assert st == 0
    ok, info = check_op_full(C, As, Bs, ta, tb, 1.0, 0.0, None, exact=True)
    assert ok, info
    if variant == "auto":
        lda, ldb = As.shape[1], Bs.shape[1]
        assert sg.sgemm_f32_ex_plan(ta, tb, M, N, K, 1.0, 256, (lda + 3) // 4 * 4, 256,
                                    (ldb + 3) // 4 * 4)[1] == sg.SKINNY


@pytest.mark.parametrize("case", [(0, 1, 16, 97, 61), (1, 1, 14, 130, 200), (0, 0, 141, 16, 61),
                                  (0, 1, 141, 7, 130), (0, 1, 16, 4096, 2500)],
                         ids=["nt", "tt", "nn-tall", "nt-tall", "nt-staged"])
def test_skinny_kmajor_odd_strides_and_beta_zero(sg, case):
    """Misaligned operands and odd strides (element-by-element loads), then
    beta = 0 over a C of NaNs, which must not be read."""
    ta, tb, M, N, K = case
    say(f"[t_skinny_kmaj_odd] {case}")
    A, B, C0 = _inputs(M, N, K, "uniform", 24)
    wa = M if ta else K
    wb = K if tb else N
    st, C, As, Bs = run_ex(sg, VID["skinny"], ta, tb, A, B, C0, 0.5, 0.25, lda=wa + 1, ldb=wb + 3,
                           ldc=N + 2, offs=(1, 3, 1))
    assert st == 0
    ok, info = check_op_full(C, As, Bs, ta, tb, 0.5, 0.25, C0)
    assert ok, info
    st, C, As, Bs = run_ex(sg, VID["skinny"], ta, tb, A, B, None, 1.0, 0.0, c_fill=np.nan)
    assert st == 0 and np.all(np.isfinite(C))
    ok, info = check_op_full(C, As, Bs, ta, tb, 1.0, 0.0, None)
    assert ok, info


def test_tensor_helper_takes_transpose_views(sg):
    M, N, K = 200, 150, 260
    A, B, C0 = _inputs(M, N, K, "uniform", 22)
    dA = torch.from_numpy(np.ascontiguousarray(A.T)).cuda()      # stored K x M
    dB = torch.from_numpy(np.ascontiguousarray(B.T)).cuda()      # stored N x K
    dC = torch.from_numpy(C0).cuda()
    sg.sgemm(dA.t(), dB.t(), dC, alpha=2.0, beta=-1.0)
    torch.cuda.synchronize()
    ok, info = check_op_full(dC.cpu().numpy(), np.ascontiguousarray(A.T), np.ascontiguousarray(B.T),
                             1, 1, 2.0, -1.0, C0)
    assert ok, info


@pytest.mark.parametrize("form", FORMS[1:], ids=FORM_IDS[1:])
def test_headline_shape_full(sg, form):
    """The 4096^3 product with alpha 1.5, beta -0.5 on N(0,1) inputs, with the
    operands stored transposed, through sgemm_f32_ex (the call the benchmark
    times for these forms)."""
    ta, tb = form
    w = workloads.WORKLOADS["square4096_ab"]
    say(f"[t_headline] {form}")
    A, B, C0 = workloads.make_inputs(w)
    As, Bs = _stored(A, ta), _stored(B, tb)
    dA = torch.from_numpy(As).cuda()
    dB = torch.from_numpy(Bs).cuda()
    dC = torch.from_numpy(C0).cuda()
    st = sg.sgemm_f32_ex(ta, tb, w.M, w.N, w.K, w.alpha, dA.data_ptr(), As.shape[1], dB.data_ptr(),
                         Bs.shape[1], w.beta, dC.data_ptr(), w.N, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    C = dC.cpu().numpy()
    assert np.all(np.isfinite(C))
    # Every element against the oracle evaluated on op(A) and op(B) themselves
    # (the same numbers, multiplied in the same k order).
    ok, info = check_full(C, A, B, w.alpha, w.beta, C0)
    assert ok, info


@pytest.mark.parametrize("form", FORMS[1:], ids=FORM_IDS[1:])
def test_ragged_full_size_integer(sg, form):
    """4092^3 integer-valued product (exact in FP32), edge tiles 252 wide on
    the 256x256 grid, every element bit for bit."""
    ta, tb = form
    say(f"[t_4092_int] {form}")
    A, B, C0 = _inputs(4092, 4092, 4092, "int4", 23)
    st, C, As, Bs = run_ex(sg, 0, ta, tb, A, B, C0, 1.0, 1.0)
    assert st == 0
    ok, info = check_full(C, A, B, 1.0, 1.0, C0, exact=True)
    assert ok, info
