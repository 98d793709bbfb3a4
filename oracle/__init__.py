"""CPU oracle for row-major FP32 GEMM, ``C = alpha*A*B + beta*C0``, and for its
form with transposed operands, ``C = alpha*op(A)*op(B) + beta*C0``.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library never imports it and
shares no code with it.

The arithmetic lives in ``sgemm_oracle.c`` (plain C, float64 accumulation, one
dot product per element in the order k = 0..K-1).  This module only marshals
numpy arrays into that library and evaluates the element-wise error bound.

Error bound for real-valued inputs.  The bound used by the checks is

    |C - Cref| <= rel * (|alpha| * (|A|*|B|)_ij + |beta| * |C0_ij|),  rel = 2e-5,

i.e. a relative tolerance of 2e-5 on the magnitude sum that an FP32 dot
product's rounding error scales with, extended with the two scaling terms.  For
integer-valued inputs whose partial sums stay below 2**24 the FP32 result is
exact in any summation order, so those checks are bit-exact against the float64
value rounded to float32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sgemm_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "liboracle.so")

REL_TOL = 2e-5

_lib = None


def compile_source(src: str, out: str) -> str:
    """Compile an oracle C source with gcc (no fast-math, no FMA contraction)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle library (always when ``force``)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    return compile_source(_SRC, _LIB_PATH)


def _bind(path: str):
    lib = ctypes.CDLL(path)
    f = ctypes.c_float
    l = ctypes.c_long
    i = ctypes.c_int
    p = ctypes.c_void_p
    lib.oracle_sgemm_f64.argtypes = [i, i, i, f, p, l, p, l, f, p, l, p, p]
    lib.oracle_sgemm_f64.restype = i
    lib.oracle_sgemm_f64_entries.argtypes = [i, i, i, f, p, l, p, l, f, p, l,
                                             l, p, p, p, p]
    lib.oracle_sgemm_f64_entries.restype = i
    lib.oracle_sgemm_op_f64.argtypes = [i, i, i, i, i, f, p, l, p, l, f, p, l, p, p]
    lib.oracle_sgemm_op_f64.restype = i
    lib.oracle_sgemm_op_f64_entries.argtypes = [i, i, i, i, i, f, p, l, p, l, f,
                                                p, l, l, p, p, p, p]
    lib.oracle_sgemm_op_f64_entries.restype = i
    lib.oracle_decode_16.argtypes = [i, p, l, p]
    lib.oracle_decode_16.restype = i
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i
    lib.oracle_set_num_threads.argtypes = [i]
    lib.oracle_set_num_threads.restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _bind(_LIB_PATH)
    return _lib


def _ld(x: np.ndarray, name: str) -> int:
    """Row stride (in elements) of a row-major float32 2-D array or view."""
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 array")
    if x.size == 0:
        return max(x.shape[1], 1)
    if x.shape[1] > 1 and x.strides[1] != 4:
        raise ValueError(f"{name} must have unit column stride")
    if x.strides[0] % 4:
        raise ValueError(f"{name} row stride must be a whole number of floats")
    return max(x.strides[0] // 4, 1)


def _ptr(x):
    return None if x is None else x.ctypes.data


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the full-matrix routines from now on (timing only)."""
    _load().oracle_set_num_threads(int(n))


def sgemm_ref(A: np.ndarray, B: np.ndarray, alpha: float = 1.0,
              beta: float = 0.0, C0: np.ndarray | None = None, _lib_override=None):
    """Full float64 product.  Returns ``(Cref, absAB)``, both M x N float64.

    ``A`` (M x K), ``B`` (K x N) and ``C0`` (M x N) are float32 arrays or
    row-major views with a row stride of at least their width.  ``C0`` is not
    read when ``beta == 0``.
    """
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    lda, ldb = _ld(A, "A"), _ld(B, "B")
    ldc = N
    if C0 is not None:
        if C0.shape != (M, N):
            raise ValueError("C0 shape")
        ldc = _ld(C0, "C0")
    elif np.float32(beta) != 0:
        raise ValueError("beta != 0 needs C0")
    Cref = np.empty((M, N), dtype=np.float64)
    absab = np.empty((M, N), dtype=np.float64)
    lib = _lib_override or _load()
    rc = lib.oracle_sgemm_f64(M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb,
                              float(beta), _ptr(C0), ldc, _ptr(Cref), _ptr(absab))
    if rc != 0:
        raise RuntimeError(f"oracle_sgemm_f64 failed with {rc}")
    return Cref, absab


def sgemm_ref_entries(A: np.ndarray, B: np.ndarray, rows, cols,
                      alpha: float = 1.0, beta: float = 0.0,
                      C0: np.ndarray | None = None, _lib_override=None):
    """Selected entries ``(rows[t], cols[t])`` of the same product.

    Returns ``(vals, absAB)`` as float64 vectors.
    """
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    lda, ldb = _ld(A, "A"), _ld(B, "B")
    ldc = N
    if C0 is not None:
        ldc = _ld(C0, "C0")
    elif np.float32(beta) != 0:
        raise ValueError("beta != 0 needs C0")
    r = np.ascontiguousarray(rows, dtype=np.int64)
    c = np.ascontiguousarray(cols, dtype=np.int64)
    if r.shape != c.shape or r.ndim != 1:
        raise ValueError("rows and cols must be equal-length vectors")
    out = np.empty(r.shape[0], dtype=np.float64)
    absab = np.empty(r.shape[0], dtype=np.float64)
    lib = _lib_override or _load()
    rc = lib.oracle_sgemm_f64_entries(M, N, K, float(alpha), _ptr(A), lda,
                                      _ptr(B), ldb, float(beta), _ptr(C0), ldc,
                                      r.shape[0], _ptr(r), _ptr(c),
                                      _ptr(out), _ptr(absab))
    if rc != 0:
        raise RuntimeError(f"oracle_sgemm_f64_entries failed with {rc}")
    return out, absab


def _op_shapes(A, B, trans_a, trans_b):
    """(M, N, K) of op(A) * op(B) for stored arrays A and B."""
    M, Ka = (A.shape[1], A.shape[0]) if trans_a else A.shape
    Kb, N = (B.shape[1], B.shape[0]) if trans_b else B.shape
    if Ka != Kb:
        raise ValueError("inner dimensions differ")
    return M, N, Ka


def _c0_ld(C0, M, N, beta, check_shape=True):
    if C0 is not None:
        if check_shape and C0.shape != (M, N):
            raise ValueError("C0 shape")
        return _ld(C0, "C0")
    if np.float32(beta) != 0:
        raise ValueError("beta != 0 needs C0")
    return max(N, 1)


def sgemm_ref_op(A: np.ndarray, B: np.ndarray, trans_a: bool = False,
                 trans_b: bool = False, alpha: float = 1.0, beta: float = 0.0,
                 C0: np.ndarray | None = None, _lib_override=None):
    """Full float64 product ``alpha * op(A) * op(B) + beta * C0``.

    ``A`` and ``B`` are the stored arrays: A is M x K, or K x M when
    ``trans_a`` (then op(A) is its transpose); B is K x N, or N x K when
    ``trans_b``.  Returns ``(Cref, absAB)``, both M x N float64.
    """
    M, N, K = _op_shapes(A, B, trans_a, trans_b)
    lda, ldb = _ld(A, "A"), _ld(B, "B")
    ldc = _c0_ld(C0, M, N, beta)
    Cref = np.empty((M, N), dtype=np.float64)
    absab = np.empty((M, N), dtype=np.float64)
    lib = _lib_override or _load()
    rc = lib.oracle_sgemm_op_f64(int(bool(trans_a)), int(bool(trans_b)), M, N, K,
                                 float(alpha), _ptr(A), lda, _ptr(B), ldb,
                                 float(beta), _ptr(C0), ldc, _ptr(Cref), _ptr(absab))
    if rc != 0:
        raise RuntimeError(f"oracle_sgemm_op_f64 failed with {rc}")
    return Cref, absab


def sgemm_ref_op_entries(A: np.ndarray, B: np.ndarray, rows, cols,
                         trans_a: bool = False, trans_b: bool = False,
                         alpha: float = 1.0, beta: float = 0.0,
                         C0: np.ndarray | None = None, _lib_override=None):
    """Selected entries ``(rows[t], cols[t])`` of ``sgemm_ref_op``'s product."""
    M, N, K = _op_shapes(A, B, trans_a, trans_b)
    lda, ldb = _ld(A, "A"), _ld(B, "B")
    ldc = _c0_ld(C0, M, N, beta, check_shape=False)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    c = np.ascontiguousarray(cols, dtype=np.int64)
    if r.shape != c.shape or r.ndim != 1:
        raise ValueError("rows and cols must be equal-length vectors")
    out = np.empty(r.shape[0], dtype=np.float64)
    absab = np.empty(r.shape[0], dtype=np.float64)
    lib = _lib_override or _load()
    rc = lib.oracle_sgemm_op_f64_entries(int(bool(trans_a)), int(bool(trans_b)), M, N, K,
                                         float(alpha), _ptr(A), lda, _ptr(B), ldb,
                                         float(beta), _ptr(C0), ldc, r.shape[0],
                                         _ptr(r), _ptr(c), _ptr(out), _ptr(absab))
    if rc != 0:
        raise RuntimeError(f"oracle_sgemm_op_f64_entries failed with {rc}")
    return out, absab


BF16 = 1
F16 = 2


def decode_16(bits: np.ndarray, kind: int, _lib_override=None) -> np.ndarray:
    """Values of 16-bit patterns (uint16 array) as float32: kind BF16 or F16."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    lib = _lib_override or _load()
    if b.size and lib.oracle_decode_16(int(kind), _ptr(b), b.size, _ptr(out)) != 0:
        raise ValueError(f"unknown 16-bit kind {kind}")
    return out


def sgemm_ref_lowp(A_bits: np.ndarray, B_bits: np.ndarray, kind: int, trans_a: bool = False,
                   trans_b: bool = False, alpha: float = 1.0, beta: float = 0.0,
                   C0: np.ndarray | None = None, _lib_override=None):
    """``alpha * op(A) * op(B) + beta * C0`` for 16-bit inputs (stored as in
    ``sgemm_ref_op``), C0 and the result float: the inputs are decoded exactly
    and multiplied by the float64 oracle.  Returns ``(Cref, absAB)``."""
    A = decode_16(A_bits, kind, _lib_override)
    B = decode_16(B_bits, kind, _lib_override)
    return sgemm_ref_op(A, B, trans_a, trans_b, alpha, beta, C0, _lib_override=_lib_override)


def sgemm_ref_lowp_entries(A_bits, B_bits, kind, rows, cols, trans_a=False, trans_b=False,
                           alpha=1.0, beta=0.0, C0=None, _lib_override=None):
    A = decode_16(A_bits, kind, _lib_override)
    B = decode_16(B_bits, kind, _lib_override)
    return sgemm_ref_op_entries(A, B, rows, cols, trans_a, trans_b, alpha, beta, C0,
                                _lib_override=_lib_override)


def error_bound(absab: np.ndarray, alpha: float, beta: float,
                c0_vals: np.ndarray | None, rel: float = REL_TOL) -> np.ndarray:
    """Element-wise bound rel * (|alpha|*absAB + |beta|*|C0|) in float64."""
    bound = abs(float(np.float32(alpha))) * np.asarray(absab, dtype=np.float64)
    if np.float32(beta) != 0 and c0_vals is not None:
        bound = bound + abs(float(np.float32(beta))) * np.abs(
            np.asarray(c0_vals, dtype=np.float64))
    return rel * bound


def check_within_bound(C: np.ndarray, Cref: np.ndarray, bound: np.ndarray):
    """Returns ``(ok, info)``; NaN or Inf anywhere in ``C`` fails."""
    C64 = np.asarray(C, dtype=np.float64)
    err = np.abs(C64 - Cref)
    bad = ~(err <= bound)  # NaN compares False, so NaN counts as bad
    n_bad = int(np.count_nonzero(bad))
    info = {"n_bad": n_bad, "max_err": float(np.nanmax(err)) if err.size else 0.0}
    if err.size:
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0),
                         np.where(err > 0, np.inf, 0.0))
        info["max_err_over_bound"] = float(np.nanmax(ratio))
    if n_bad:
        idx = np.argwhere(bad.reshape(C64.shape) if C64.ndim else bad)[0]
        info["first_bad_index"] = tuple(int(v) for v in np.atleast_1d(idx))
    return n_bad == 0, info


def check_bitexact(C: np.ndarray, Cref: np.ndarray):
    """Bit-exact comparison of a float32 result with float32(Cref)."""
    want = np.asarray(Cref, dtype=np.float64).astype(np.float32)
    got = np.asarray(C, dtype=np.float32)
    diff = got.view(np.uint32) != want.view(np.uint32)
    n_bad = int(np.count_nonzero(diff))
    info = {"n_bad": n_bad}
    if n_bad:
        idx = np.argwhere(diff)[0]
        info["first_bad_index"] = tuple(int(v) for v in np.atleast_1d(idx))
        info["got"] = float(got[tuple(idx)])
        info["want"] = float(want[tuple(idx)])
    return n_bad == 0, info


class BoundOracle:
    """The same API bound to another compiled copy of the oracle source.

    Used only by the tests that plant a mistake in a copy of the oracle and
    check that the pins catch it.
    """

    def __init__(self, lib_path: str):
        self._lib = _bind(lib_path)

    def sgemm_ref(self, A, B, alpha=1.0, beta=0.0, C0=None):
        return sgemm_ref(A, B, alpha, beta, C0, _lib_override=self._lib)

    def sgemm_ref_entries(self, A, B, rows, cols, alpha=1.0, beta=0.0, C0=None):
        return sgemm_ref_entries(A, B, rows, cols, alpha, beta, C0,
                                 _lib_override=self._lib)

    def decode_16(self, bits, kind):
        return decode_16(bits, kind, _lib_override=self._lib)

    def sgemm_ref_lowp(self, A_bits, B_bits, kind, trans_a=False, trans_b=False, alpha=1.0,
                       beta=0.0, C0=None):
        return sgemm_ref_lowp(A_bits, B_bits, kind, trans_a, trans_b, alpha, beta, C0,
                              _lib_override=self._lib)

    def sgemm_ref_op(self, A, B, trans_a=False, trans_b=False, alpha=1.0, beta=0.0, C0=None):
        return sgemm_ref_op(A, B, trans_a, trans_b, alpha, beta, C0, _lib_override=self._lib)

    def sgemm_ref_op_entries(self, A, B, rows, cols, trans_a=False, trans_b=False,
                             alpha=1.0, beta=0.0, C0=None):
        return sgemm_ref_op_entries(A, B, rows, cols, trans_a, trans_b, alpha, beta, C0,
                                    _lib_override=self._lib)


SOURCE_PATH = _SRC
