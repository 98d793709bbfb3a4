"""Helpers for the GPU tests: run the library through its C interface on
seeded inputs and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle


def dev():
    return torch.device("cuda:0")


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device_padded(X: np.ndarray | None, ld: int, offset: int = 0, fill=np.nan):
    """Copies a host matrix into a device buffer with row stride ``ld`` and the
    first element ``offset`` floats past the buffer start.  Returns
    (buffer, pointer, ld)."""
    rows, cols = X.shape
    total = offset + (rows - 1) * ld + cols if rows > 0 else offset + 1
    host = np.full(max(total, 1), fill, dtype=np.float32)
    if rows > 0 and cols > 0:
        view = np.lib.stride_tricks.as_strided(host[offset:], shape=(rows, cols),
                                               strides=(ld * 4, 4))
        view[...] = X
    buf = torch.from_numpy(host).to(dev())
    return buf, buf.data_ptr() + 4 * offset, ld


def from_device_padded(buf, rows: int, cols: int, ld: int, offset: int = 0) -> np.ndarray:
    host = buf.cpu().numpy()
    if rows == 0 or cols == 0:
        return np.zeros((rows, cols), np.float32)
    view = np.lib.stride_tricks.as_strided(host[offset:], shape=(rows, cols), strides=(ld * 4, 4))
    return np.array(view)


VECTOR_ONLY = (1, 2)   # mfma_large, mfma_small


def run_lib(sg, variant, A, B, C0, alpha, beta, lda=None, ldb=None, ldc=None,
            offs=(0, 0, 0), c_fill=np.nan, stream=None):
    """Runs sgemm_f32_variant on host inputs; returns (status, C, Cbuf_host).

    C0 = None with beta == 0 leaves C's initial contents at ``c_fill``.
    """
    M, K = A.shape
    N = B.shape[1]
    # The vector-load variants need row strides that are multiples of 4 floats;
    # give them padded strides unless the test chose its own.
    r4 = (lambda x: (max(x, 1) + 3) // 4 * 4) if variant in VECTOR_ONLY else (lambda x: max(x, 1))
    lda = lda or r4(K)
    ldb = ldb or r4(N)
    ldc = ldc or max(N, 1)
    bA, pA, _ = to_device_padded(A, lda, offs[0])
    bB, pB, _ = to_device_padded(B, ldb, offs[1])
    Cinit = C0 if C0 is not None else np.full((M, N), c_fill, np.float32)
    bC, pC, _ = to_device_padded(Cinit, ldc, offs[2], fill=np.float32(-7.25))
    s = stream or torch.cuda.current_stream(dev())
    st = sg.sgemm_f32_variant(variant, M, N, K, float(alpha), pA, lda, pB, ldb, float(beta),
                              pC, ldc, s.cuda_stream)
    torch.cuda.synchronize(dev())
    Cbuf = bC.cpu().numpy()
    C = from_device_padded(bC, M, N, ldc, offs[2])
    return st, C, Cbuf


def check_full(C, A, B, alpha, beta, C0, exact=False):
    Cref, absab = oracle.sgemm_ref(A, B, alpha, beta, C0)
    if exact:
        return oracle.check_bitexact(C, Cref)
    bound = oracle.error_bound(absab, alpha, beta, C0)
    return oracle.check_within_bound(C, Cref, bound)


def zero_sum_integers(M, N, K, seed):
    """Integer-valued operands (values -4..4) whose product has exactly zero
    entries: row 1 of A is zero, column 2 of B is zero, and (where the shape
    allows) entry (0, 0) cancels (A[0, 0:2] = 1, 1 and B[0:2, 0] = 3, -3, the
    rest of row 0 of A zero).  With alpha < 0 and beta = 0 those entries are
    alpha * (+0) = -0 in IEEE arithmetic."""
    rng = np.random.default_rng(seed)
    A = rng.integers(-4, 5, (M, K)).astype(np.float32)
    B = rng.integers(-4, 5, (K, N)).astype(np.float32)
    if M > 1:
        A[1, :] = 0
    if N > 2:
        B[:, 2] = 0
    if K >= 2:
        A[0, :] = 0
        A[0, :2] = 1
        B[:2, 0] = [3, -3]
    return A, B


def sample_positions(M, N, n_random, seed, full_rows=2, full_cols=2):
    """Random entries plus whole rows and columns (first/last included)."""
    rng = np.random.default_rng(seed)
    rows = [rng.integers(0, M, n_random)]
    cols = [rng.integers(0, N, n_random)]
    pick_r = sorted(set([0, M - 1] + list(rng.integers(0, M, max(full_rows - 2, 0)))))
    pick_c = sorted(set([0, N - 1] + list(rng.integers(0, N, max(full_cols - 2, 0)))))
    for r in pick_r:
        rows.append(np.full(N, r))
        cols.append(np.arange(N))
    for c in pick_c:
        rows.append(np.arange(M))
        cols.append(np.full(M, c))
    return np.concatenate(rows).astype(np.int64), np.concatenate(cols).astype(np.int64)


def check_sampled(C, A, B, alpha, beta, C0, rows, cols, exact=False):
    vals, absab = oracle.sgemm_ref_entries(A, B, rows, cols, alpha, beta, C0)
    got = C[rows, cols]
    if exact:
        return oracle.check_bitexact(got, vals)
    c0v = None if C0 is None else C0[rows, cols]
    bound = oracle.error_bound(absab, alpha, beta, c0v)
    return oracle.check_within_bound(got, vals, bound)


def check_row_col_sums(C, A, B, alpha, beta, C0, rel=2e-5):
    """Whole-matrix property: row and column sums of C equal those of
    alpha*A*B + beta*C0, formed from matrix-vector products in float64."""
    A64 = A.astype(np.float64)
    B64 = B.astype(np.float64)
    C64 = C.astype(np.float64)
    aA, aB = np.abs(A64), np.abs(B64)
    rs_want = alpha * (A64 @ B64.sum(axis=1))
    rs_mag = abs(alpha) * (aA @ aB.sum(axis=1))
    cs_want = alpha * (A64.sum(axis=0) @ B64)
    cs_mag = abs(alpha) * (aA.sum(axis=0) @ aB)
    if beta != 0 and C0 is not None:
        C064 = C0.astype(np.float64)
        rs_want = rs_want + beta * C064.sum(axis=1)
        rs_mag = rs_mag + abs(beta) * np.abs(C064).sum(axis=1)
        cs_want = cs_want + beta * C064.sum(axis=0)
        cs_mag = cs_mag + abs(beta) * np.abs(C064).sum(axis=0)
    rs_err = np.abs(C64.sum(axis=1) - rs_want)
    cs_err = np.abs(C64.sum(axis=0) - cs_want)
    ok = bool(np.all(rs_err <= rel * rs_mag + 1e-9) and np.all(cs_err <= rel * cs_mag + 1e-9))
    return ok, {"row_sum_worst": float(np.max(rs_err / np.maximum(rel * rs_mag, 1e-300))),
                "col_sum_worst": float(np.max(cs_err / np.maximum(rel * cs_mag, 1e-300)))}
