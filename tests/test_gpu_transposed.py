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


@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
def test_beta_zero_ignores_nan_c(sg, form):
    ta, tb = form
    A, B, _ = _inputs(150, 140, 90, "uniform", 20, c0=False)
    st, C, As, Bs = run_ex(sg, 0, ta, tb, A, B, None, 1.0, 0.0, c_fill=np.nan)
    assert st == 0 and np.all(np.isfinite(C))
    ok, info = check_op_full(C, As, Bs, ta, tb, 1.0, 0.0, None)
    assert ok, info


@pytest.mark.parametrize("form", FORMS[1:], ids=FORM_IDS[1:])
def test_unsupported_variants_refuse(sg, form):
    ta, tb = form
    A, B, C0 = _inputs(16, 64, 64, "uniform", 21)
    for v in ("valu", "skinny"):
        st, _, _, _ = run_ex(sg, VID[v], ta, tb, A, B, C0, 1.0, 0.0)
        assert st == sg.ERR_NOT_APPLICABLE, v


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
