"""Python binding of the gfx950 FP32 GEMM library (``libsgemm_f32.so``).

Argument marshalling only: every step of ``C = alpha*op(A)*op(B) + beta*C``
runs in the library's HIP kernels.  The functions mirror the C interface in
``include/sgemm_f32.h`` one to one (same names, same argument order, device
pointers passed as integers, status codes returned unchanged).  ``sgemm``
adds a convenience form over PyTorch tensors, which serve only as device memory
and streams.

Importing this package loads the library; if it has not been built the import
fails with an error rather than falling back to any other implementation.
"""
from __future__ import annotations

import ctypes
import os

from . import _build

LIB_PATH = _build.LIB_PATH

AUTO = 0
MFMA_LARGE = 1
MFMA_SMALL = 2
VALU = 3
SKINNY = 4
MFMA_SCALAR = 5
MFMA_TUNED = 6
NUM_VARIANTS = 7

CFG_128x128 = 0
CFG_64x64 = 1
CFG_128x64 = 2
CFG_64x128 = 3
CFG_64x64_PF2 = 4
CFG_128x128_STREAMK = 5
CFG_64x64_BK64 = 6
CFG_256x256 = 7
CFG_128x128_DL = 8
CFG_64x64_DL = 9
CFG_192x192_DL = 10
NUM_CONFIGS = 11

ERR_VARIANT = 20
ERR_NOT_APPLICABLE = 21
ERR_TOO_LARGE = 22
ERR_TRANS = 23
ERR_CONFIG = 24
ERR_SCRATCH = 25
NOALLOC_SCRATCH_BYTES = 64 << 20

GEMM16_BF16 = 1
GEMM16_F16 = 2
GEMM16_ERR_ALIGN = 21
GEMM16_ERR_TYPE = 25

EXPORTED = ("sgemm_f32", "sgemm_f32_noalloc", "sgemm_f32_variant", "sgemm_f32_select",
            "sgemm_f32_ex", "sgemm_f32_ex_variant", "sgemm_f32_ex_select",
            "sgemm_f32_ex_plan", "sgemm_f32_ex_config", "sgemm_f32_config_name",
            "sgemm_f32_tuning_table_present", "sgemm_f32_variant_name", "sgemm_f32_version",
            "gemm16_f32")


class SgemmError(RuntimeError):
    def __init__(self, status: int, what: str = "sgemm_f32"):
        super().__init__(f"{what} returned status {status}")
        self.status = status


def _load_library(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    i, f, p = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    gemm_args = [i, i, i, f, p, i, p, i, f, p, i, p]
    lib.sgemm_f32.argtypes = gemm_args
    lib.sgemm_f32.restype = i
    lib.sgemm_f32_noalloc.argtypes = gemm_args
    lib.sgemm_f32_noalloc.restype = i
    lib.sgemm_f32_variant.argtypes = [i] + gemm_args
    lib.sgemm_f32_variant.restype = i
    lib.sgemm_f32_select.argtypes = [i, i, i, f, p, i, p, i]
    lib.sgemm_f32_select.restype = i
    lib.sgemm_f32_ex.argtypes = [i, i] + gemm_args
    lib.sgemm_f32_ex.restype = i
    lib.sgemm_f32_ex_variant.argtypes = [i, i, i] + gemm_args
    lib.sgemm_f32_ex_variant.restype = i
    lib.sgemm_f32_ex_select.argtypes = [i, i, i, i, i, f, p, i, p, i]
    lib.sgemm_f32_ex_select.restype = i
    ip = ctypes.POINTER(ctypes.c_int)
    lib.sgemm_f32_ex_plan.argtypes = [i, i, i, i, i, f, p, i, p, i, ip, ip, ip, ip]
    lib.sgemm_f32_ex_plan.restype = i
    lib.sgemm_f32_ex_config.argtypes = [i, i, i, i, i] + gemm_args
    lib.sgemm_f32_ex_config.restype = i
    lib.sgemm_f32_config_name.argtypes = [i]
    lib.sgemm_f32_config_name.restype = ctypes.c_char_p
    lib.sgemm_f32_tuning_table_present.argtypes = []
    lib.sgemm_f32_tuning_table_present.restype = i
    lib.gemm16_f32.argtypes = [i, i, i] + gemm_args
    lib.gemm16_f32.restype = i
    lib.sgemm_f32_variant_name.argtypes = [i]
    lib.sgemm_f32_variant_name.restype = ctypes.c_char_p
    lib.sgemm_f32_version.argtypes = []
    lib.sgemm_f32_version.restype = i
    return lib


_lib = _load_library()


def lds_poison_library():
    """The LDS-poisoning debug copy of the library (its kernels fill their LDS
    with NaN before the first load), bound with the same C signatures; for the
    tests that check that no LDS stage is read before it is filled."""
    return _load_library(_build.POISON_LIB_PATH)

_INT_MIN, _INT_MAX = -(1 << 31), (1 << 31) - 1


def _ints(*vals) -> None:
    """ctypes wraps an out-of-range int silently (K = 2**32 + 5 would arrive as 5),
    so every integer argument of the C interface is range-checked first."""
    for v in vals:
        if not _INT_MIN <= int(v) <= _INT_MAX:
            raise OverflowError(f"{v} does not fit the C interface's 32-bit int")


def sgemm_f32(M: int, N: int, K: int, alpha: float, A: int, lda: int, B: int, ldb: int,
              beta: float, C: int, ldc: int, stream: int = 0) -> int:
    """The C entry point: raw device pointers and a hipStream_t as integers."""
    _ints(M, N, K, lda, ldb, ldc)
    return _lib.sgemm_f32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def sgemm_f32_noalloc(M: int, N: int, K: int, alpha: float, A: int, lda: int, B: int, ldb: int,
                      beta: float, C: int, ldc: int, stream: int = 0) -> int:
    """sgemm_f32 with no device allocation: split plans use the library's fixed
    per-device scratch region (calls that overlap on one device race on it)."""
    _ints(M, N, K, lda, ldb, ldc)
    return _lib.sgemm_f32_noalloc(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def sgemm_f32_variant(variant: int, M: int, N: int, K: int, alpha: float, A: int, lda: int,
                      B: int, ldb: int, beta: float, C: int, ldc: int, stream: int = 0) -> int:
    _ints(variant, M, N, K, lda, ldb, ldc)
    return _lib.sgemm_f32_variant(variant, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def sgemm_f32_select(M: int, N: int, K: int, alpha: float, A: int, lda: int, B: int,
                     ldb: int) -> int:
    _ints(M, N, K, lda, ldb)
    return _lib.sgemm_f32_select(M, N, K, alpha, A, lda, B, ldb)


def sgemm_f32_ex(trans_a: int, trans_b: int, M: int, N: int, K: int, alpha: float, A: int,
                 lda: int, B: int, ldb: int, beta: float, C: int, ldc: int, stream: int = 0) -> int:
    """C = alpha*op(A)*op(B) + beta*C; a flag of 1 means the operand is stored transposed."""
    _ints(trans_a, trans_b, M, N, K, lda, ldb, ldc)
    return _lib.sgemm_f32_ex(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def sgemm_f32_ex_variant(variant: int, trans_a: int, trans_b: int, M: int, N: int, K: int,
                         alpha: float, A: int, lda: int, B: int, ldb: int, beta: float, C: int,
                         ldc: int, stream: int = 0) -> int:
    _ints(variant, trans_a, trans_b, M, N, K, lda, ldb, ldc)
    return _lib.sgemm_f32_ex_variant(variant, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb,
                                     beta, C, ldc, stream)


def sgemm_f32_ex_select(trans_a: int, trans_b: int, M: int, N: int, K: int, alpha: float,
                        A: int, lda: int, B: int, ldb: int) -> int:
    _ints(trans_a, trans_b, M, N, K, lda, ldb)
    return _lib.sgemm_f32_ex_select(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb)


def sgemm_f32_ex_plan(trans_a: int, trans_b: int, M: int, N: int, K: int, alpha: float, A: int,
                      lda: int, B: int, ldb: int):
    """Returns (status, variant, config, group_m, splits) of the automatic choice."""
    _ints(trans_a, trans_b, M, N, K, lda, ldb)
    out = [ctypes.c_int(0) for _ in range(4)]
    st = _lib.sgemm_f32_ex_plan(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb,
                                *[ctypes.byref(o) for o in out])
    return (st,) + tuple(o.value for o in out)


def sgemm_f32_ex_config(config: int, group_m: int, splits: int, trans_a: int, trans_b: int, M: int,
                        N: int, K: int, alpha: float, A: int, lda: int, B: int, ldb: int, beta: float,
                        C: int, ldc: int, stream: int = 0) -> int:
    _ints(config, group_m, splits, trans_a, trans_b, M, N, K, lda, ldb, ldc)
    return _lib.sgemm_f32_ex_config(config, group_m, splits, trans_a, trans_b, M, N, K, alpha, A, lda,
                                    B, ldb, beta, C, ldc, stream)


def sgemm_f32_config_name(config: int) -> str | None:
    _ints(config)
    r = _lib.sgemm_f32_config_name(config)
    return None if r is None else r.decode()


def sgemm_f32_tuning_table_present() -> int:
    return _lib.sgemm_f32_tuning_table_present()


def gemm16_f32(in_type: int, trans_a: int, trans_b: int, M: int, N: int, K: int, alpha: float, A: int,
               lda: int, B: int, ldb: int, beta: float, C: int, ldc: int, stream: int = 0) -> int:
    """C (float) = alpha*op(A)*op(B) + beta*C with A, B of 16-bit values
    (GEMM16_BF16 or GEMM16_F16 bit patterns), FP32 accumulation."""
    _ints(in_type, trans_a, trans_b, M, N, K, lda, ldb, ldc)
    return _lib.gemm16_f32(in_type, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def sgemm_f32_variant_name(variant: int) -> str | None:
    _ints(variant)
    r = _lib.sgemm_f32_variant_name(variant)
    return None if r is None else r.decode()


def sgemm_f32_version() -> int:
    return _lib.sgemm_f32_version()


def _check_tensor(t, name: str) -> None:
    import torch

    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _row_stride(t, name: str) -> int:
    _check_tensor(t, name)
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must be row-major with unit column stride")
    return max(int(t.stride(0)), 1) if t.shape[0] > 1 else max(int(t.shape[1]), 1)


def _operand(t, name: str):
    """(leading dimension, transpose flag) of an operand view.

    A row-major view is passed as stored (flag 0).  A view with unit row stride
    is the transpose of a row-major matrix (``X.t()``), passed as that stored
    matrix with flag 1.
    """
    _check_tensor(t, name)
    rows, cols = int(t.shape[0]), int(t.shape[1])
    if cols <= 1 or t.stride(1) == 1:
        return (max(int(t.stride(0)), 1) if rows > 1 else max(cols, 1)), 0
    if rows <= 1 or t.stride(0) == 1:
        return (max(int(t.stride(1)), 1) if cols > 1 else max(rows, 1)), 1
    raise ValueError(f"{name} must be row-major or the transpose of a row-major matrix")


def sgemm(A, B, C, alpha: float = 1.0, beta: float = 0.0, variant: int = AUTO,
          stream=None) -> None:
    """C = alpha*A@B + beta*C in place on device tensors.

    ``A`` and ``B`` may each be a row-major view or the transpose view of one
    (``X.t()``); the latter is passed to the library as a transposed operand.
    ``C`` must be row-major.  ``stream`` is a ``torch.cuda.Stream`` (default:
    the current stream).  The call is asynchronous on that stream.  Raises
    ``SgemmError`` on a non-zero status.
    """
    import torch

    M, K = A.shape
    K2, N = B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    lda, ta = _operand(A, "A")
    ldb, tb = _operand(B, "B")
    ldc = _row_stride(C, "C")
    if A.device != C.device or B.device != C.device:
        raise ValueError(f"A, B and C must be on one device: {A.device}, {B.device}, {C.device}")
    if stream is None:
        stream = torch.cuda.current_stream(C.device)
    # The library launches on the current device (and keeps its workspace per
    # device), so C's device is made current for the call.
    with torch.cuda.device(C.device):
        st = sgemm_f32_ex_variant(variant, ta, tb, M, N, K, float(alpha), A.data_ptr(), lda,
                                  B.data_ptr(), ldb, float(beta), C.data_ptr(), ldc,
                                  stream.cuda_stream)
    if st != 0:
        raise SgemmError(st)
