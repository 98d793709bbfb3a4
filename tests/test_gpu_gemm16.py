"""GPU parity of the 16-bit-input GEMM (gemm16_f32) against the oracle's
16-bit-input form: the same 16-bit patterns decoded exactly and multiplied in
float64.  Real-valued inputs within 2e-5 * (|alpha|*(|op(A)||op(B)|)_ij +
|beta|*|C0_ij|) per element; integer-valued inputs (exact products and sums)
bit for bit.  Both formats, all four operand forms, the in-place (NT,
aligned, K a multiple of 64) and the packed paths."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import from_device_padded, say, to_device_padded

pytestmark = pytest.mark.gpu

FORMS = [(0, 0), (0, 1), (1, 0), (1, 1)]
FORM_IDS = ["nn", "nt", "tn", "tt"]
KINDS = [1, 2]
KIND_IDS = ["bf16", "f16"]


@pytest.fixture(scope="module")
def sg():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import fp32_sgemm_amd
    return fp32_sgemm_amd


def _stored(x, t):
    return np.ascontiguousarray(x.T) if t else x


def _dev16(X, ld, offset=0):
    """Copies a uint16 host matrix into a device buffer with row stride ld and
    the first element `offset` elements in; returns (buffer, pointer)."""
    rows, cols = X.shape
    total = offset + (rows - 1) * ld + cols if rows > 0 else offset + 1
    host = np.full(max(total, 1), 0x7FC0, dtype=np.uint16)      # NaN patterns around the matrix
    if rows and cols:
        np.lib.stride_tricks.as_strided(host[offset:], shape=(rows, cols), strides=(ld * 2, 2))[...] = X
    buf = torch.from_numpy(host.view(np.int16)).cuda()
    return buf, buf.data_ptr() + 2 * offset


def run16(sg, kind, ta, tb, A, B, C0, alpha, beta, pad=(0, 0), offs=(0, 0), c_fill=np.nan, ldc=None):
    """A (M x K) and B (K x N) are op(A) and op(B) as uint16 patterns."""
    M, K = A.shape
    N = B.shape[1]
    As, Bs = _stored(A, ta), _stored(B, tb)
    lda, ldb = max(As.shape[1], 1) + pad[0], max(Bs.shape[1], 1) + pad[1]
    ldc = max(N, 1) if ldc is None else ldc
    bA, pA = _dev16(As, lda, offs[0])
    bB, pB = _dev16(Bs, ldb, offs[1])
    Cinit = C0 if C0 is not None else np.full((M, N), c_fill, np.float32)
    bC, pC, _ = to_device_padded(Cinit, ldc, fill=np.float32(-7.25))
    st = sg.gemm16_f32(kind, ta, tb, M, N, K, float(alpha), pA, lda, pB, ldb, float(beta), pC, ldc,
                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    if ldc > N and M > 1:
        # The gap between one row of C and the next is left alone.
        gap = bC[N:N + (M - 1) * ldc].view(M - 1, ldc)[:, :ldc - N].cpu().numpy()
        assert np.all(gap == np.float32(-7.25)), "C written between its rows"
    return st, from_device_padded(bC, M, N, ldc), As, Bs


def _inputs16(M, N, K, dist, kind, seed):
    w = workloads.custom(M, N, K, dist=dist, seed=seed, c0_dist="normal" if dist != "int4" else "int4")
    return workloads.make_inputs_16bit(w, kind)


def check16_logical(C, A, B, kind, alpha, beta, C0, exact):
    """Every element against the float64 oracle on op(A) and op(B) themselves
    (A, B: the 16-bit patterns of the operands as they enter the product,
    decoded exactly), for the large shapes."""
    Cref, absab = oracle.sgemm_ref(oracle.decode_16(A, kind), oracle.decode_16(B, kind),
                                   alpha, beta, C0)
    if exact:
        return oracle.check_bitexact(C, Cref)
    return oracle.check_within_bound(C, Cref, oracle.error_bound(absab, alpha, beta, C0))


def check16(C, As, Bs, kind, ta, tb, alpha, beta, C0, exact):
    Cref, absab = oracle.sgemm_ref_lowp(As, Bs, kind, ta, tb, alpha, beta, C0)
    if exact:
        return oracle.check_bitexact(C, Cref)
    return oracle.check_within_bound(C, Cref, oracle.error_bound(absab, alpha, beta, C0))


SHAPES = [(1, 1, 1), (17, 31, 33), (129, 127, 65), (300, 260, 700), (128, 128, 128), (64, 64, 64),
          (257, 129, 1000), (130, 70, 9), (256, 256, 4096), (200, 136, 192)]


@pytest.mark.parametrize("kind", KINDS, ids=KIND_IDS)
@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
def test_gemm16_real(sg, kind, form, shape):
    M, N, K = shape
    ta, tb = form
    say(f"[g16_real] kind={kind} {form} {shape}")
    A, B, C0 = _inputs16(M, N, K, "uniform", kind, 1500 + M + N + K)
    st, C, As, Bs = run16(sg, kind, ta, tb, A, B, C0, 1.25, -0.5)
    assert st == 0
    ok, info = check16(C, As, Bs, kind, ta, tb, 1.25, -0.5, C0, exact=False)
    assert ok, info


@pytest.mark.parametrize("kind", KINDS, ids=KIND_IDS)
@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
def test_gemm16_integer_bitexact(sg, kind, form, shape):
    M, N, K = shape
    ta, tb = form
    say(f"[g16_int] kind={kind} {form} {shape}")
    A, B, C0 = _inputs16(M, N, K, "int4", kind, 1600 + M + N + K)
    st, C, As, Bs = run16(sg, kind, ta, tb, A, B, C0, 2.0, -1.0)
    assert st == 0
    ok, info = check16(C, As, Bs, kind, ta, tb, 2.0, -1.0, C0, exact=True)
    assert ok, info


@pytest.mark.parametrize("kind", KINDS, ids=KIND_IDS)
def test_gemm16_misaligned_and_padded_strides(sg, kind):
    """NT with strides that are not multiples of 8 and pointers off 16 bytes:
    the packed path."""
    M, N, K = 150, 90, 256
    A, B, C0 = _inputs16(M, N, K, "uniform", kind, 41)
    st, C, As, Bs = run16(sg, kind, 0, 1, A, B, C0, 0.5, 0.25, pad=(3, 5), offs=(1, 3))
    assert st == 0
    ok, info = check16(C, As, Bs, kind, 0, 1, 0.5, 0.25, C0, exact=False)
    assert ok, info


@pytest.mark.parametrize("kind", KINDS, ids=KIND_IDS)
@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("K", [200, 256])
def test_gemm16_c_stride_past_32bit_tile_offsets(sg, kind, form, K):
    """ldc = 2,200,000: a 256-row tile of C would span more than 2 GiB, past
    the direct-to-LDS kernel's 32-bit epilogue offsets, so the register-staged
    kernel (64-bit C offsets) takes the product, here on 5 rows of C (K = 256
    with NT reads the operands in place, the other cases pack them first);
    the gaps between the rows stay untouched."""
    M, N = 5, 300
    ta, tb = form
    say(f"[g16_wide_ldc] kind={kind} {form} K={K}")
    A, B, C0 = _inputs16(M, N, K, "int4", kind, 1700 + K + 2 * ta + tb)
    st, C, As, Bs = run16(sg, kind, ta, tb, A, B, C0, 1.0, -1.0, ldc=2_200_000)
    assert st == 0
    ok, info = check16(C, As, Bs, kind, ta, tb, 1.0, -1.0, C0, exact=True)
    assert ok, info


@pytest.mark.parametrize("kind", KINDS, ids=KIND_IDS)
@pytest.mark.parametrize("shape", [(140, 130, 128), (3072, 3000, 128), (4096, 4096, 128), (16, 4096, 4096)],
                         ids=["tile128", "tile192", "tile256", "split_k"])
def test_gemm16_beta_zero_ignores_nan_c(sg, kind, shape):
    """beta = 0: C is written without being read (NaN there stays out of the
    result) on each tile size of the direct-to-LDS kernel."""
    M, N, K = shape
    A, B, _ = _inputs16(M, N, K, "uniform", kind, 42)
    st, C, As, Bs = run16(sg, kind, 0, 1, A, B, None, 1.0, 0.0, c_fill=np.nan)
    assert st == 0 and np.all(np.isfinite(C))
    ok, info = check16(C, As, Bs, kind, 0, 1, 1.0, 0.0, None, exact=False)
    assert ok, info


def test_gemm16_alpha_zero_and_k_zero(sg):
    M, N = 70, 90
    C0 = np.random.default_rng(3).standard_normal((M, N)).astype(np.float32)
    A = np.full((M, 30), 0x7FC0, np.uint16)
    B = np.full((30, N), 0x7FC0, np.uint16)
    st, C, _, _ = run16(sg, 1, 0, 0, A, B, C0, 0.0, -0.5)
    assert st == 0 and np.array_equal(C, np.float32(-0.5) * C0)
    st, C, _, _ = run16(sg, 2, 0, 1, np.zeros((M, 0), np.uint16), np.zeros((0, N), np.uint16), C0, 2.0, 3.0)
    assert st == 0 and np.array_equal(C, np.float32(3.0) * C0)


@pytest.mark.parametrize("kind", KINDS, ids=KIND_IDS)
@pytest.mark.parametrize("form", [(0, 1), (0, 0), (1, 1)], ids=["nt", "nn", "tt"])
def test_gemm16_headline_shape(sg, kind, form):
    """4096^3 with alpha 1.5, beta -0.5 on N(0,1) inputs stored in 16 bits,
    every operand read in place by the larger-tile kernel (A transposed and B
    as given through transposing LDS reads)."""
    ta, tb = form
    w = workloads.WORKLOADS["square4096_ab"]
    say(f"[g16_headline] kind={kind} {form}")
    A, B, C0 = workloads.make_inputs_16bit(w, kind)
    st, C, As, Bs = run16(sg, kind, ta, tb, A, B, C0, w.alpha, w.beta)
    assert st == 0 and np.all(np.isfinite(C))
    ok, info = check16_logical(C, A, B, kind, w.alpha, w.beta, C0, exact=False)
    assert ok, info


@pytest.mark.parametrize("kind", KINDS, ids=KIND_IDS)
def test_gemm16_ragged_large_integer(sg, kind):
    M, N, K = 4092, 3000, 4100
    A, B, C0 = _inputs16(M, N, K, "int4", kind, 43)
    st, C, As, Bs = run16(sg, kind, 1, 0, A, B, C0, 1.0, 1.0)
    assert st == 0
    ok, info = check16_logical(C, A, B, kind, 1.0, 1.0, C0, exact=True)
    assert ok, info


@pytest.mark.parametrize("kind", KINDS, ids=KIND_IDS)
@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
def test_gemm16_big_tiles_with_edges(sg, kind, form):
    """A grid of 256 tiles of 256 x 256 (the larger tile) whose M and N are
    not tile multiples (edge tiles 160 and 120 wide), beta != 0 (the edge
    epilogue reads and writes C through the buffer resource), every element
    checked."""
    ta, tb = form
    M, N, K = 4000, 3960, 256
    say(f"[g16_big_edges] kind={kind} {form}")
    A, B, C0 = _inputs16(M, N, K, "uniform", kind, 45 + 2 * ta + tb)
    st, C, As, Bs = run16(sg, kind, ta, tb, A, B, C0, 1.5, -0.5)
    assert st == 0 and np.all(np.isfinite(C))
    ok, info = check16_logical(C, A, B, kind, 1.5, -0.5, C0, exact=False)
    assert ok, info


@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("kind", KINDS, ids=KIND_IDS)
def test_gemm16_big_tiles_integer_bitexact(sg, kind, form):
    """K = 576 (a multiple of 64): the larger-tile kernel reads A transposed
    and B as given in place (transposing LDS reads); M = 3832 and N = 3904
    (240 tiles of 256 x 256) leave a row of edge tiles 248 high and a column
    64 wide."""
    M, N, K = 3832, 3904, 576
    ta, tb = form
    A, B, C0 = _inputs16(M, N, K, "int4", kind, 47)
    st, C, As, Bs = run16(sg, kind, ta, tb, A, B, C0, 1.0, -1.0)
    assert st == 0
    ok, info = check16_logical(C, A, B, kind, 1.0, -1.0, C0, exact=True)
    assert ok, info


@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("kind", KINDS, ids=KIND_IDS)
@pytest.mark.parametrize("shape", [(2900, 3000, 576), (3072, 3072, 64), (2880, 2888, 1000)],
                         ids=["edges", "one_slice", "ragged_k"])
def test_gemm16_192_tiles_bitexact(sg, kind, form, shape):
    """Grids of 224 to 256 tiles of 192 x 192 (and fewer than 256 of
    256 x 256) run the direct-to-LDS kernel on 192 x 192 tiles, whose rows of
    k along x are 384 bytes with their own rotation: edge tiles in M and N,
    a single slice, and K = 1000 (packed, padded to 1024)."""
    M, N, K = shape
    ta, tb = form
    say(f"[g16_192] kind={kind} {form} {shape}")
    A, B, C0 = _inputs16(M, N, K, "int4", kind, 80 + K + 2 * ta + tb)
    st, C, As, Bs = run16(sg, kind, ta, tb, A, B, C0, 1.0, -1.0)
    assert st == 0
    ok, info = check16_logical(C, A, B, kind, 1.0, -1.0, C0, exact=True)
    assert ok, info


@pytest.mark.parametrize("kind", KINDS, ids=KIND_IDS)
@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
def test_gemm16_192_tiles_real(sg, kind, form):
    """3072^3 with alpha 1.5, beta -0.5 on N(0,1) inputs: 256 tiles of
    192 x 192, every element within the bound."""
    ta, tb = form
    M = N = K = 3072
    say(f"[g16_192_real] kind={kind} {form}")
    w = workloads.custom(M, N, K, dist="normal", seed=91, c0_dist="normal")
    A, B, C0 = workloads.make_inputs_16bit(w, kind)
    st, C, As, Bs = run16(sg, kind, ta, tb, A, B, C0, 1.5, -0.5)
    assert st == 0 and np.all(np.isfinite(C))
    ok, info = check16_logical(C, A, B, kind, 1.5, -0.5, C0, exact=False)
    assert ok, info


SPLIT_SHAPES = [(16, 4096, 4096), (1, 1000, 2048), (64, 2048, 8192)]


@pytest.mark.parametrize("kind", KINDS, ids=KIND_IDS)
@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SPLIT_SHAPES])
def test_gemm16_split_k(sg, kind, form, shape):
    """Grids of few 128 x 128 tiles split K over work-groups (8 or 16
    splits here): partial tiles in the call's scratch, added in split order
    by a second kernel, which applies alpha and beta.  Integer inputs bit for
    bit, real inputs within the bound."""
    M, N, K = shape
    ta, tb = form
    say(f"[g16_split] kind={kind} {form} {shape}")
    A, B, C0 = _inputs16(M, N, K, "int4", kind, 90 + M + 2 * ta + tb)
    st, C, As, Bs = run16(sg, kind, ta, tb, A, B, C0, 1.0, -1.0)
    assert st == 0
    ok, info = check16_logical(C, A, B, kind, 1.0, -1.0, C0, exact=True)
    assert ok, info
    A, B, C0 = _inputs16(M, N, K, "normal", kind, 95 + M + 2 * ta + tb)
    st, C, As, Bs = run16(sg, kind, ta, tb, A, B, C0, 1.5, -0.5)
    assert st == 0 and np.all(np.isfinite(C))
    ok, info = check16_logical(C, A, B, kind, 1.5, -0.5, C0, exact=False)
    assert ok, info


@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("K", [8, 64, 192])
def test_gemm16_big_tiles_short_k_bitexact(sg, K, form):
    """The larger-tile kernel loads B one 64-deep slice ahead and A two;
    with one to three slices (K padded to 64, or 192) the first and last
    slices' special cases (no A two ahead, nothing to load) all run."""
    M, N = 4096, 4096
    ta, tb = form
    say(f"[g16_big_short_k] K={K} {form}")
    A, B, C0 = _inputs16(M, N, K, "int4", 1, 60 + K)
    st, C, As, Bs = run16(sg, 1, ta, tb, A, B, C0, 1.0, -1.0)
    assert st == 0
    ok, info = check16_logical(C, A, B, 1, 1.0, -1.0, C0, exact=True)
    assert ok, info


@pytest.mark.parametrize("kind", KINDS, ids=KIND_IDS)
@pytest.mark.parametrize("shape", [(150, 140, 96), (3072, 3072, 64), (4096, 4096, 64), (16, 2048, 2048)],
                         ids=["small_grid", "tile192", "big_tiles", "split_k"])
def test_gemm16_negative_alpha_zero_sums_bitexact(sg, kind, shape):
    """alpha < 0 with beta = 0: exactly zero sums are alpha * (+0) = -0, the
    oracle's value, on each tile size of the direct-to-LDS kernel."""
    from gpu_helpers import zero_sum_integers
    M, N, K = shape
    say(f"[g16_neg_alpha_zero] kind={kind} {shape}")
    Af, Bf = zero_sum_integers(M, N, K, 72)
    A, B = workloads.to_16bit(Af, kind), workloads.to_16bit(Bf, kind)
    st, C, _, _ = run16(sg, kind, 0, 1, A, B, None, -1.0, 0.0, c_fill=np.nan)
    assert st == 0
    assert np.all(np.signbit(C[1, :])) and np.all(C[1, :] == 0)
    ok, info = check16_logical(C, A, B, kind, -1.0, 0.0, None, exact=True)
    assert ok, info
