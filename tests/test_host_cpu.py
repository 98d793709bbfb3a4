"""CPU-only checks: the C library loads and exports what its header declares,
host-side argument handling and kernel selection, the tile mapping, the
benchmark's closed-form work/byte model, and the input generators.  No GPU
compute is launched here."""
from __future__ import annotations

import glob
import os
import re
import shutil
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgemm_f32.h")


HEADERS = sorted(glob.glob(os.path.join(os.path.dirname(HEADER), "*.h")))


def _declared_functions():
    names = set()
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def sg():
    import fp32_sgemm_amd
    return fp32_sgemm_amd


def test_header_declares_the_interface():
    names = _declared_functions()
    assert {"sgemm_f32", "sgemm_f32_variant", "sgemm_f32_select", "sgemm_f32_variant_name",
            "sgemm_f32_version", "gemm16_f32"} <= set(names), names
    assert len(HEADERS) == 2, HEADERS


def test_library_exports_every_declared_symbol(sg):
    out = subprocess.run(["nm", "-D", "--defined-only", sg.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, flags=re.M))
    for name in _declared_functions():
        assert name in exported, f"{name} declared in include/ but not exported"
        assert hasattr(sg._lib, name)
    assert set(sg.EXPORTED) == set(_declared_functions())


def test_library_loads_after_torch():
    """In a process that imported torch first, the library's HIP symbols bind
    to the HIP runtime torch brings (an older one than the system's), so the
    library may only use entry points that runtime has; a newer one fails the
    load.  Run in a fresh process to fix the import order."""
    code = ("import torch, fp32_sgemm_amd as sg; "
            "assert sg.sgemm_f32_version() > 0; print('ok')")
    p = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert p.returncode == 0 and "ok" in p.stdout, p.stderr[-2000:]


def test_lds_poison_copy_exports_the_same_interface(sg):
    """The debug copy that the LDS-poisoning GPU tests run is built from the
    same sources and exports every declared function too."""
    from fp32_sgemm_amd import _build
    out = subprocess.run(["nm", "-D", "--defined-only", _build.POISON_LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, flags=re.M))
    assert set(_declared_functions()) <= exported


@pytest.mark.parametrize("src,kernels", [("sgemm_big.hip", 24), ("gemm16.hip", 26)])
def test_lds_poison_flag_fills_lds_with_nan(tmp_path, src, kernels):
    """The debug flag really plants the NaN fill: the device code of the
    kernels built with SGEMM_LDS_POISON holds the quiet-NaN constant once per
    LDS-using kernel instance (4 tile sizes x 4 operand forms of the
    direct-to-LDS kernel, plus its two-group 64x64 and 128x128 forms x 4; in the 16-bit
    GEMM, the register-staged 128 x 128 kernel x 2 formats and the
    direct-to-LDS kernel x 3 tile sizes x 2 formats x A and B each K-major or
    read along x), and the product build holds none."""
    from fp32_sgemm_amd import _build
    counts = []
    for extra in (["-DSGEMM_LDS_POISON=1"], []):
        out = tmp_path / f"{src}{len(extra)}.s"
        cmd = [_build.HIPCC, *_build.COMMON_FLAGS, *extra, "--cuda-device-only", "-S", "-o", str(out),
               os.path.join(_build.CSRC, src)]
        subprocess.run(cmd, check=True, capture_output=True)
        counts.append(out.read_text().count("0x7fc00000"))
    assert counts == [kernels, 0], counts


def test_binding_mirrors_the_c_names(sg):
    for name in _declared_functions():
        assert callable(getattr(sg, name)), name


def test_argument_errors_without_touching_the_gpu(sg):
    p = 0x1000  # never dereferenced: every call below fails validation first
    f = sg.sgemm_f32
    assert f(-1, 2, 2, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == 1
    assert f(2, -1, 2, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == 2
    assert f(2, 2, -1, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == 3
    assert f(2, 2, 2, 1.0, 0, 2, p, 2, 0.0, p, 2, 0) == 5
    assert f(2, 2, 3, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == 6
    assert f(2, 2, 2, 1.0, p, 2, 0, 2, 0.0, p, 2, 0) == 7
    assert f(2, 3, 2, 1.0, p, 2, p, 2, 0.0, p, 3, 0) == 8
    assert f(2, 2, 2, 1.0, p, 2, p, 2, 0.0, 0, 2, 0) == 10
    assert f(2, 3, 2, 1.0, p, 2, p, 3, 0.0, p, 2, 0) == 11
    assert f(2, 2, 0, 1.0, 0, 1, 0, 2, 0.0, 0, 2, 0) == 10   # K = 0 still writes C
    assert sg.sgemm_f32_variant(-1, 2, 2, 2, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == sg.ERR_VARIANT
    assert sg.sgemm_f32_variant(sg.NUM_VARIANTS, 2, 2, 2, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == sg.ERR_VARIANT


def test_binding_rejects_ints_that_ctypes_would_wrap(sg):
    # 2**32 + 5 would reach the library as 5 and silently compute another product.
    p = 0x1000
    with pytest.raises(OverflowError):
        sg.sgemm_f32(2, 2, 2**32 + 5, 1.0, p, 2**32 + 5, p, 2, 0.0, p, 2, 0)
    with pytest.raises(OverflowError):
        sg.sgemm_f32_ex(0, 0, 2, 2, 2, 1.0, p, 2, p, 2**31, 0.0, p, 2, 0)
    with pytest.raises(OverflowError):
        sg.sgemm_f32_ex_config(0, 8, 1, 0, 0, -(2**31) - 1, 2, 2, 1.0, p, 2, p, 2, 0.0, p, 2, 0)
    with pytest.raises(OverflowError):
        sg.gemm16_f32(sg.GEMM16_BF16, 0, 0, 2, 2**31, 2, 1.0, p, 2, p, 2, 0.0, p, 2, 0)
    assert sg.sgemm_f32(2**31 - 1, 2, 2, 1.0, 0, 2, p, 2, 0.0, p, 2, 0) == 5   # in range: C checks


def test_empty_outputs_return_without_work(sg):
    # M == 0 or N == 0: success without any launch (NULL pointers are fine).
    assert sg.sgemm_f32(0, 5, 7, 1.0, 0, 7, 0, 5, 0.0, 0, 5, 0) == 0
    assert sg.sgemm_f32(5, 0, 7, 1.0, 0, 7, 0, 1, 0.0, 0, 1, 0) == 0


def test_kernel_selection(sg):
    al = 0x100000          # 16-byte aligned stand-in pointers (never dereferenced)
    # 4096^3: whole 256x256 tiles filling one round (configuration 7, reported as the tuned plan)
    assert sg.sgemm_f32_select(4096, 4096, 4096, 1.5, al, 4096, al, 4096) == sg.MFMA_TUNED
    assert sg.sgemm_f32_select(4092, 4092, 4092, 1.0, al, 4092, al, 4092) == sg.MFMA_TUNED
    assert sg.sgemm_f32_select(3000, 3000, 3000, 1.0, al, 3000, al, 3000) == sg.MFMA_TUNED
    # Shapes with few 128x128 tiles: the small tile, or the tuning table's plan.
    assert sg.sgemm_f32_select(1024, 1024, 1024, 1.0, al, 1024, al, 1024) in (sg.MFMA_SMALL, sg.MFMA_TUNED)
    assert sg.sgemm_f32_select(128, 128, 128, 1.0, al, 128, al, 128) in (sg.MFMA_SMALL, sg.MFMA_TUNED)
    assert sg.sgemm_f32_select(16, 4096, 4096, 1.0, al, 4096, al, 4096) == sg.SKINNY
    assert sg.sgemm_f32_select(32, 4096, 4096, 1.0, al, 4096, al, 4096) == sg.SKINNY   # two blocks of 16 rows
    assert sg.sgemm_f32_select(33, 4096, 4096, 1.0, al, 4096, al, 4096) != sg.SKINNY
    # A misaligned A of 64 MiB is copied to aligned rows and takes the 256x256
    # tiles; one past the copies' 64 MiB keeps the 4-byte loads.
    assert sg.sgemm_f32_ex_plan(0, 0, 4096, 4096, 4096, 1.0, al + 4, 4096, al, 4096)[1:3] == \
        (sg.MFMA_TUNED, sg.CFG_256x256)
    assert sg.sgemm_f32_select(4097, 4096, 4096, 1.0, al + 4, 4096, al, 4096) == sg.MFMA_SCALAR
    assert sg.sgemm_f32_select(4096, 4096, 4097, 1.0, al, 4097, al, 4096) == sg.MFMA_SCALAR
    assert sg.sgemm_f32_select(4096, 4096, 4096, 0.0, al, 4096, al, 4096) == 0
    assert sg.sgemm_f32_select(4096, 4096, 0, 1.0, al, 1, al, 4096) == 0


def test_transposed_argument_errors_without_touching_the_gpu(sg):
    p = 0x1000
    f = sg.sgemm_f32_ex
    # Flags other than 0 and 1.
    assert f(2, 0, 2, 2, 2, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == sg.ERR_TRANS
    assert f(0, -1, 2, 2, 2, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == sg.ERR_TRANS
    # A stored K x M when transposed: lda >= M; B stored N x K: ldb >= K.
    assert f(1, 0, 5, 2, 3, 1.0, p, 4, p, 2, 0.0, p, 2, 0) == 6      # lda 4 < M 5
    assert f(0, 1, 2, 5, 3, 1.0, p, 3, p, 2, 0.0, p, 5, 0) == 8      # ldb 2 < K 3
    assert f(0, 1, 2, 5, 3, 1.0, p, 3, p, 3, 0.0, p, 4, 0) == 11     # ldc 4 < N 5
    # The widths the untransposed forms would need are not required.
    assert f(1, 1, 2, 5, 9, 1.0, p, 2, p, 9, 0.0, 0, 5, 0) == 10     # only C is missing
    assert sg.sgemm_f32_ex_variant(sg.NUM_VARIANTS, 1, 0, 2, 2, 2, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == sg.ERR_VARIANT
    # The VALU kernel takes neither operand transposed; the streaming kernels
    # take every form but A transposed with B as given, and A transposed
    # when only N is small.
    al = 0x100000
    for ta, tb in ((1, 0), (0, 1), (1, 1)):
        assert sg.sgemm_f32_ex_variant(sg.VALU, ta, tb, 16, 64, 64, 1.0, al, 64, al, 64, 0.0, al, 64, 0) \
            == sg.ERR_NOT_APPLICABLE, (ta, tb)
    assert sg.sgemm_f32_ex_variant(sg.SKINNY, 1, 0, 16, 64, 64, 1.0, al, 64, al, 64, 0.0, al, 64, 0) \
        == sg.ERR_NOT_APPLICABLE
    for tb in (0, 1):
        assert sg.sgemm_f32_ex_variant(sg.SKINNY, 1, tb, 64, 16, 64, 1.0, al, 64, al, 64, 0.0, al, 64, 0) \
            == sg.ERR_NOT_APPLICABLE, tb
        assert sg.sgemm_f32_ex_variant(sg.SKINNY, 0, tb, 64, 17, 64, 1.0, al, 64, al, 64, 0.0, al, 64, 0) \
            == sg.ERR_NOT_APPLICABLE, tb
    for ta in (0, 1):
        assert sg.sgemm_f32_ex_variant(sg.SKINNY, ta, 1, 17, 64, 64, 1.0, al, 64, al, 64, 0.0, al, 64, 0) \
            == sg.ERR_NOT_APPLICABLE, ta
    assert sg.sgemm_f32_ex_variant(sg.SKINNY, 0, 0, 33, 33, 64, 1.0, al, 64, al, 64, 0.0, al, 64, 0) \
        == sg.ERR_NOT_APPLICABLE


def test_transposed_kernel_selection(sg):
    al = 0x100000
    sel = sg.sgemm_f32_ex_select
    for ta, tb in ((0, 1), (1, 0), (1, 1)):
        assert sel(ta, tb, 4096, 4096, 4096, 1.0, al, 4096, al, 4096) == sg.MFMA_TUNED
        # configuration 8 wherever its operand conditions hold
        assert sel(ta, tb, 6144, 6144, 2048, 1.0, al, 6144 if ta else 2048, al, 2048 if tb else 6144) \
            == sg.MFMA_TUNED
        assert sg.sgemm_f32_ex_plan(ta, tb, 6144, 6144, 2048, 1.0, al, 6144 if ta else 2048, al,
                                    2048 if tb else 6144)[2] == sg.CFG_128x128_DL
        assert sg.sgemm_f32_ex_plan(ta, tb, 7000, 7000, 1024, 1.0, al, 7000 if ta else 1024, al,
                                    1024 if tb else 7000)[2] == sg.CFG_128x128_DL
        assert sg.sgemm_f32_ex_plan(ta, tb, 7000, 7000, 1000, 1.0, al, 7000 if ta else 1000, al,
                                    1000 if tb else 7000)[2] == sg.CFG_128x128_DL
        assert sel(ta, tb, 1024, 1024, 1024, 1.0, al, 1024, al, 1024) in (sg.MFMA_SMALL, sg.MFMA_TUNED)
        # M <= 16 with B given N x K streams B along k; A transposed with B as
        # given stays on tiles.
        assert sel(ta, tb, 16, 4096, 4096, 1.0, al, 4096, al, 4096) == \
            (sg.SKINNY if tb else sg.MFMA_TUNED)
        assert sel(ta, tb, 1, 4096, 4096, 1.0, al, 4096, al, 4096) == \
            (sg.SKINNY if tb else sg.MFMA_TUNED)
        assert sel(ta, tb, 17, 4096, 4096, 1.0, al, 4096, al, 4096) != sg.SKINNY
        # N <= 16 with A as given streams A along k (C written transposed).
        assert sel(ta, tb, 4096, 16, 4096, 1.0, al, 4096, al, 4096) == \
            (sg.MFMA_TUNED if ta else sg.SKINNY)
        assert sel(ta, tb, 4096, 17, 4096, 1.0, al, 4096, al, 4096) != sg.SKINNY
        # An odd stride of A: copied to aligned rows when the copy fits in
        # 64 MiB, 4-byte loads beyond.
        assert sel(ta, tb, 4096, 4096, 4096, 1.0, al, 4097, al, 4096) == sg.MFMA_TUNED
        assert sel(ta, tb, 4096, 4096, 4100, 1.0, al, 4101, al, 4100) == sg.MFMA_SCALAR
    assert sel(0, 0, 16, 4096, 4096, 1.0, al, 4096, al, 4096) == sg.SKINNY
    assert sel(0, 0, 4096, 16, 4096, 1.0, al, 4096, al, 16) == sg.SKINNY
    assert sel(0, 0, 4096, 1, 4096, 1.0, al, 4096, al, 1) == sg.SKINNY
    # The streamed operand's 32 rows, and all of the small one, must lie within
    # 32-bit byte offsets: B's stride too wide for 32 rows keeps the tiles.
    wide = (1 << 31) // 4 // 31 + 4
    assert sel(0, 1, 16, 4096, 4096, 1.0, al, 4096, al, wide - wide % 4) != sg.SKINNY
    assert sel(0, 1, 16, 4096, 4096, 1.0, al, 4096, al, (1 << 31) // 4 // 32 - 1024) == sg.SKINNY
    # A given K x M (k-major) spans K rows of its stride.
    assert sel(1, 1, 16, 4096, 65536, 1.0, al, 16384, al, 65536) != sg.SKINNY
    assert sel(0, 0, 4096, 4096, 4096, 1.0, al, 4096, al, 4096) == \
        sg.sgemm_f32_select(4096, 4096, 4096, 1.0, al, 4096, al, 4096)
    assert sel(2, 0, 4096, 4096, 4096, 1.0, al, 4096, al, 4096) == 0
    # 2 GiB rule: an operand stored along K spans 128 rows per slice, one
    # stored along M or N 32 rows.
    big = (1 << 31) // 4 // 100          # 128 rows of this stride exceed 2 GiB, 32 rows do not
    assert sel(0, 0, 4096, 4096, 4100, 1.0, al, big - big % 4, al, 4096) == sg.MFMA_SCALAR
    # ... unless the rows fit in 64 MiB once copied to aligned rows of their own.
    assert sel(0, 0, 4096, 4096, 4096, 1.0, al, big - big % 4, al, 4096) == sg.MFMA_TUNED
    # A stored transposed (along M): 16-byte loads; the 256x256 tiles read 16 of its rows per slice.
    ld = big - big % 4
    assert sel(1, 0, 4096, 4096, 4096, 1.0, al, ld, al, 4096) == sg.MFMA_TUNED
    assert sg.sgemm_f32_ex_plan(1, 0, 4096, 4096, 4096, 1.0, al, ld, al, 4096)[2] == sg.CFG_256x256
    assert sel(1, 0, 4094, 4092, 4092, 1.0, al, ld, al, 4092) == sg.MFMA_LARGE


def test_gemm16_argument_errors_without_touching_the_gpu(sg):
    p = 0x1000
    f = sg.gemm16_f32
    assert f(0, 0, 1, 2, 2, 2, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == sg.GEMM16_ERR_TYPE
    assert f(3, 0, 1, 2, 2, 2, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == sg.GEMM16_ERR_TYPE
    assert f(1, 2, 1, 2, 2, 2, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == sg.ERR_TRANS
    assert f(1, 0, 1, -1, 2, 2, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == 1
    assert f(1, 0, 1, 2, 2, 2, 1.0, 0, 2, p, 2, 0.0, p, 2, 0) == 5
    assert f(1, 0, 1, 2, 2, 3, 1.0, p, 2, p, 3, 0.0, p, 2, 0) == 6          # A is 2 x 3: lda >= 3
    assert f(1, 0, 1, 2, 5, 3, 1.0, p, 3, p, 2, 0.0, p, 5, 0) == 8          # B stored 5 x 3: ldb >= 3
    assert f(2, 0, 0, 2, 5, 3, 1.0, p, 3, p, 4, 0.0, p, 5, 0) == 8          # B stored 3 x 5: ldb >= 5
    assert f(1, 0, 1, 2, 2, 2, 1.0, p, 2, p, 2, 0.0, 0, 2, 0) == 10
    assert f(1, 0, 1, 2, 2, 2, 1.0, p + 1, 2, p, 2, 0.0, p, 2, 0) == sg.GEMM16_ERR_ALIGN
    assert f(1, 0, 1, 2, 2, 4000001, 1.0, p, 4000001, p, 4000001, 0.0, p, 2, 0) == sg.ERR_TOO_LARGE
    assert f(1, 0, 1, 0, 2, 2, 1.0, 0, 2, 0, 2, 0.0, 0, 2, 0) == 0          # empty output


def test_variant_names_and_version(sg):
    names = [sg.sgemm_f32_variant_name(i) for i in range(sg.NUM_VARIANTS)]
    assert names == ["auto", "mfma_large", "mfma_small", "valu", "skinny", "mfma_scalar", "mfma_tuned"]
    assert sg.sgemm_f32_variant_name(sg.NUM_VARIANTS) is None
    cfgs = [sg.sgemm_f32_config_name(i) for i in range(sg.NUM_CONFIGS)]
    assert cfgs == ["128x128", "64x64", "128x64", "64x128", "64x64_pf2", "128x128_streamk", "64x64_bk64", "256x256",
                    "128x128_dl", "64x64_dl", "192x192_dl"]
    assert sg.sgemm_f32_config_name(sg.NUM_CONFIGS) is None and sg.sgemm_f32_config_name(-1) is None
    assert sg.sgemm_f32_version() >= 300


def test_config_and_plan_argument_errors_without_touching_the_gpu(sg):
    p = 0x1000
    f = sg.sgemm_f32_ex_config
    for bad in [(-1, 8, 1), (sg.NUM_CONFIGS, 8, 1), (0, 0, 1), (0, 65, 1), (0, 8, 0), (0, 8, 65)]:
        assert f(*bad, 0, 0, 2, 2, 2, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == sg.ERR_CONFIG, bad
    assert f(0, 8, 1, 0, 0, -1, 2, 2, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == 1
    assert f(0, 8, 1, 3, 0, 2, 2, 2, 1.0, p, 2, p, 2, 0.0, p, 2, 0) == sg.ERR_TRANS
    assert f(0, 8, 1, 0, 0, 2, 2, 2, 1.0, p, 2, p, 2, 0.0, 0, 2, 0) == 10
    assert f(0, 8, 1, 0, 0, 0, 2, 2, 1.0, 0, 2, 0, 2, 0.0, 0, 2, 0) == 0        # empty output
    # The 16-byte-only configurations refuse misaligned operands before any launch.
    for cfg in (2, 3, 4, 5):
        assert f(cfg, 8, 1, 0, 0, 64, 64, 64, 1.0, p + 4, 64, p, 64, 0.0, p, 64, 0) == sg.ERR_NOT_APPLICABLE
    # The persistent configuration takes no split count.
    assert f(5, 8, 2, 0, 0, 64, 64, 64, 1.0, p, 64, p, 64, 0.0, p, 64, 0) == sg.ERR_CONFIG
    # A split plan whose partials exceed 1 GiB is refused before any launch.
    assert f(0, 8, 64, 0, 0, 8192, 8192, 8192, 1.0, p, 8192, p, 8192, 0.0, p, 8192, 0) == sg.ERR_TOO_LARGE
    assert sg.sgemm_f32_ex_plan(2, 0, 4, 4, 4, 1.0, p, 4, p, 4)[0] == sg.ERR_TRANS
    assert sg.sgemm_f32_ex_plan(0, 0, 4, -4, 4, 1.0, p, 4, p, 4)[0] == 2
    assert sg.sgemm_f32_ex_plan(0, 0, 4, 4, 0, 1.0, p, 4, p, 4) == (0, 0, 0, 0, 0)


def test_config6_needs_64_rows_within_2gib(sg):
    """Configuration 6 stages 64 values of k per slice: an operand stored along
    N (B as given) whose 64 rows span 2 GiB or more is refused (no launch),
    where the 32-row configurations still run."""
    al = 0x100000
    big_ldb = 10_000_000          # 31 rows fit in 2 GiB of offsets, 63 do not
    st = sg.sgemm_f32_ex_config(6, 8, 1, 0, 0, 64, 64, 64, 1.0, al, 64, al, big_ldb, 0.0, al, 64, 0)
    assert st == sg.ERR_NOT_APPLICABLE
    st = sg.sgemm_f32_ex_config(6, 8, 1, 1, 0, 64, 64, 64, 1.0, al, big_ldb, al, 64, 0.0, al, 64, 0)
    assert st == sg.ERR_NOT_APPLICABLE


def test_small_tiles_for_poorly_filled_rounds(sg):
    """128x128 grids of at least 256 tiles that fill less than 0.88 of their
    rounds of 512 resident work-groups (a single partial round included) move
    to 64x64 tiles with two slices in flight; well-filled grids keep 128x128."""
    al = 0x100000
    plan = lambda M, N, K, ta=0, tb=0: sg.sgemm_f32_ex_plan(ta, tb, M, N, K, 1.0, al, M if ta else K, al,
                                                            K if tb else N)
    # 64x64 tiles: loaded straight into LDS (configuration 9) when the grid has
    # at most 1024 tiles (one round), edge tiles included, else
    # with two slices in flight.
    for shape in [(3500, 3500, 3500), (5000, 5000, 1000), (4608, 4608, 2048),
                  (7168, 7168, 1024), (2048, 2560, 2048), (2304, 2304, 4096), (2048, 3072, 1024),
                  (2560, 2560, 2560), (3072, 2880, 2048), (3072, 3072, 512)]:
        assert plan(*shape)[1:] == (sg.MFMA_TUNED, sg.CFG_64x64_PF2, 8, 1), shape
    # One round of 250 to 256 tiles of 192x192 (K >= 1024), or whole rounds in
    # place of 64x64 tiles: configuration 10.
    for shape in [(3000, 3000, 3000), (3008, 3008, 3008), (3072, 3072, 1024), (2976, 2976, 2976),
                  (1536, 6144, 4096), (2880, 3264, 2048), (6144, 3072, 2048), (4608, 6144, 2048),
                  (9216, 3072, 2048), (3072, 9216, 1024)]:
        assert plan(*shape)[1:] == (sg.MFMA_TUNED, sg.CFG_192x192_DL, 8, 1), shape
    assert plan(4608, 4608, 4096)[2] == sg.CFG_64x64_PF2      # 2.25 rounds
    assert plan(6144, 6144, 4096)[2] == sg.CFG_128x128_DL     # four rounds, well-filled 128x128 grid
    assert plan(6144, 3072, 512)[2] != sg.CFG_192x192_DL      # short K
    for shape in [(2048, 2048, 2048), (2048, 2048, 1024), (2048, 2048, 4096), (2048, 2048, 2044)]:
        assert plan(*shape)[1:3] == (sg.MFMA_TUNED, sg.CFG_128x128_DL), shape
    # Edge tiles (M, N multiples of 4): the 64x64 direct-to-LDS grid, here one
    # round of 128x128 tiles in turn.
    assert plan(2040, 2048, 2048)[1:3] == (sg.MFMA_TUNED, sg.CFG_128x128_DL)
    assert plan(500, 2000, 4096)[1:3] == (sg.MFMA_TUNED, sg.CFG_64x64_DL)
    # N not a multiple of 4 with B as given: K split on one round of 64x64 tiles.
    assert sg.sgemm_f32_ex_plan(0, 0, 512, 2047, 4096, 1.0, al, 4096, al, 2048)[1:] == (sg.MFMA_TUNED, 4, 8, 3)
    assert sg.sgemm_f32_ex_plan(0, 0, 2048, 1023, 2048, 1.0, al, 2048, al, 1024)[4] == 2
    assert sg.sgemm_f32_ex_plan(0, 0, 1024, 1023, 1024, 1.0, al, 1024, al, 1024)[4] == 1
    assert sg.sgemm_f32_ex_plan(0, 1, 512, 2047, 4096, 1.0, al, 4096, al, 4096)[4] == 1
    # An unevenly spread 64x64 grid that cannot take the direct-to-LDS tiles (M
    # odd): split as configuration 9 grids are.
    assert plan(131, 6000, 2048)[1:] == (sg.MFMA_TUNED, 4, 8, 3)
    assert plan(2001, 1000, 1600)[4] == 1
    # 64x64 grids spread unevenly over the CUs (1.2 times the mean or more)
    # with K >= 1536: back to configuration 4 with K split in 2 or 3.
    for shape, splits in [((1152, 1152, 4096), 3), ((1280, 1280, 2048), 3), ((1536, 1536, 4096), 3),
                          ((1792, 1792, 4096), 3), ((1600, 1600, 4096), 2), ((1536, 1024, 4096), 2),
                          ((1536, 1536, 1536), 3), ((1600, 1600, 1600), 2)]:
        assert plan(*shape)[1:] == (sg.MFMA_TUNED, sg.CFG_64x64_PF2, 8, splits), shape
    for shape in [(1280, 1280, 1280), (1408, 1408, 4096), (1664, 1664, 4096), (256, 4096, 4096),
                  (2048, 2048, 512)]:
        assert plan(*shape)[1:] == (sg.MFMA_TUNED, sg.CFG_64x64_DL, 8, 1), shape
    # A configuration 9 grid that is one round of 128x128 tiles (K >= 1024):
    # configuration 8.
    for shape in [(2048, 2048, 2048), (1024, 4096, 4096), (4096, 1024, 4096), (2048, 2048, 1024)]:
        assert plan(*shape)[1:] == (sg.MFMA_TUNED, sg.CFG_128x128_DL, 8, 1), shape
    assert plan(3000, 3000, 3000, 1, 1)[1:3] == (sg.MFMA_TUNED, sg.CFG_192x192_DL)
    assert plan(3000, 3002, 3000)[1:3] != (sg.MFMA_TUNED, sg.CFG_192x192_DL)   # N of B as given not a multiple of 4
    assert plan(3002, 3000, 3000)[1:3] == (sg.MFMA_TUNED, sg.CFG_192x192_DL)   # M of A as given: rows read as zero
    for shape in [(6144, 6144, 2048), (4096, 11008, 512), (10240, 10240, 1024), (2816, 2816, 2816)]:
        assert plan(*shape)[2] == sg.CFG_128x128_DL, shape
    for shape in [(7000, 7000, 1024), (7040, 7000, 1024), (10000, 10000, 1024)]:
        assert plan(*shape)[2] == sg.CFG_128x128_DL, shape
    for shape in [(7040, 7040, 1000), (7000, 7000, 1000)]:
        assert plan(*shape)[2] == sg.CFG_128x128_DL, shape
    # N of B as given not a multiple of 4: the register-staged 128x128 kernel;
    # M of A as given may be anything.
    assert plan(7000, 7002, 1024)[1:3] == (sg.MFMA_LARGE, sg.CFG_128x128)
    assert plan(7002, 7000, 1024)[1:3] == (sg.MFMA_TUNED, sg.CFG_128x128_DL)
    # Well-filled 256x256 grids take the larger tile.
    for shape in [(4096, 4096, 4096), (8192, 8192, 8192), (4092, 4092, 4092)]:
        assert plan(*shape)[2] == sg.CFG_256x256, shape
    # The persistent stream-K configuration is never chosen automatically.
    for shape in [(3000, 3000, 3000), (2900, 4100, 2048), (5000, 5000, 1000)]:
        assert plan(*shape)[2] != sg.CFG_128x128_STREAMK, shape
    # 4-byte loads keep their kernel where the aligned copy would exceed 64 MiB.
    st, v, cfg, gm, sp = sg.sgemm_f32_ex_plan(0, 0, 4100, 4100, 4101, 1.0, al, 4101, al, 4100)
    assert (v, cfg) == (sg.MFMA_SCALAR, 0)
    assert sg.sgemm_f32_ex_plan(0, 0, 3000, 3000, 3001, 1.0, al, 3001, al, 3000)[1] == sg.MFMA_TUNED


def test_plan_follows_the_tuning_table(sg):
    """The automatic plan for aligned operands is the tuning table's entry of
    the shape class (or the default choice when no table is compiled in)."""
    import json
    import os
    al = 0x100000
    st, v, cfg, gm, sp = sg.sgemm_f32_ex_plan(0, 0, 16, 4096, 4096, 1.0, al, 4096, al, 4096)
    assert (st, v) == (0, sg.SKINNY)
    st, v, cfg, gm, sp = sg.sgemm_f32_ex_plan(0, 0, 4096, 4096, 4097, 1.0, al, 4097, al, 4096)
    assert (st, v, sp) == (0, sg.MFMA_SCALAR, 1)
    # Few tiles with 4-byte loads: K split to about 512 work-groups, each split
    # at least 256 deep.
    assert sg.sgemm_f32_ex_plan(0, 0, 4096, 17, 4096, 1.0, al, 4096, al, 17) == (0, sg.MFMA_SCALAR, 1, 8, 8)
    assert sg.sgemm_f32_ex_plan(0, 0, 1000, 33, 3001, 1.0, al, 3001, al, 36)[4] == 11
    assert sg.sgemm_f32_ex_plan(0, 0, 64, 64, 511, 1.0, al, 511, al, 64)[4] == 1
    # Many tiles with 4-byte loads: operands copied to aligned rows first when
    # the copies fit in 64 MiB and the product is at least 2^32 FLOP; the plan
    # reported is the one that then runs.
    assert sg.sgemm_f32_ex_plan(0, 0, 2047, 2047, 2047, 1.0, al, 2047, al, 2047) == \
        (0, sg.MFMA_TUNED, sg.CFG_64x64_PF2, 8, 1)
    assert sg.sgemm_f32_ex_plan(1, 1, 1700, 1500, 1600, 1.0, al, 1701, al, 1601)[1] == sg.MFMA_TUNED
    assert sg.sgemm_f32_ex_plan(0, 0, 1023, 1023, 1023, 1.0, al, 1023, al, 1023)[1] == sg.MFMA_SCALAR
    assert sg.sgemm_f32_ex_plan(0, 0, 4095, 4095, 4095, 1.0, al, 4095, al, 4095)[1] == sg.MFMA_SCALAR
    path = os.path.join(os.path.dirname(sg.__file__), "tuning_table.json")
    if not sg.sgemm_f32_tuning_table_present():
        assert not os.path.exists(path)
        for shape in [(4096, 4096, 4096), (2048, 2048, 2048), (1024, 1024, 1024)]:
            st, v, cfg, gm, sp = sg.sgemm_f32_ex_plan(0, 0, *shape, 1.0, al, shape[2], al, shape[1])
            assert (v, cfg) in ((sg.MFMA_LARGE, sg.CFG_128x128), (sg.MFMA_TUNED, sg.CFG_64x64_PF2))
            assert gm == 8 and sp == 1
        return
    table = json.load(open(path))
    bounds = table["class_bounds"]
    assert bounds == [64, 128, 256, 512, 1024, 2048, 4096, 8192]
    for e in table["entries"]:
        M, N, K = e["shape"]
        st, v, cfg, gm, sp = sg.sgemm_f32_ex_plan(0, 0, M, N, K, 1.0, al, K, al, N)
        if M <= 32 or N <= 16:
            assert v == sg.SKINNY
            continue
        assert st == 0 and v in (sg.MFMA_LARGE, sg.MFMA_SMALL, sg.MFMA_TUNED), e
        if cfg in (sg.CFG_64x64_PF2, sg.CFG_64x64_DL) and e["config"] == 0:
            continue        # the switch to 64x64 tiles for poorly filled rounds
        if cfg in (sg.CFG_256x256, sg.CFG_128x128_DL) and e["config"] == 0 and e["splits"] == 1:
            continue        # 256x256 tiles, or the 128x128 grid loaded straight into LDS
        if cfg == sg.CFG_64x64_DL and e["config"] in (0, 4) and e["splits"] == 1:
            continue        # the 64x64 grid loaded straight into LDS
        assert (cfg, gm) == (e["config"], e["group_m"]), e
        k_per = -(-K // e["splits"])
        k_per = -(-k_per // 32) * 32
        assert sp == -(-K // k_per), e
        # Every extent in the class maps to the same entry.
        st2, v2, cfg2, gm2, sp2 = sg.sgemm_f32_ex_plan(0, 0, M - 1 if M > 64 else M, N, K, 1.0, al, K, al, N)
        assert (cfg2, gm2) == (cfg, gm)





def test_tile_mapping_is_a_bijection(tmp_path):
    exe = tmp_path / "tile_map_check"
    src = os.path.join(ROOT, "tests", "host", "tile_map_check.cpp")
    inc = os.path.join(ROOT, "fp32_sgemm_amd", "csrc")
    subprocess.run(["/opt/rocm/bin/hipcc", "-x", "hip", "--offload-arch=gfx950", "-O1",
                    "-I", inc, src, "-o", str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout


def test_build_flags_disable_packed_fp32():
    from fp32_sgemm_amd import _build
    flags = " ".join(_build.COMMON_FLAGS)
    assert "-target-feature -Xclang -packed-fp32-ops" in flags
    assert "--offload-arch=gfx950" in flags
    assert "fast-math" not in flags


def test_product_package_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "fp32_sgemm_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "oracle" not in text.lower(), f"{fn} mentions the oracle"


def test_missing_library_fails_loudly(tmp_path):
    """A copy of the package without its built library must refuse to import."""
    dst = tmp_path / "fp32_sgemm_amd"
    shutil.copytree(os.path.join(ROOT, "fp32_sgemm_amd"), dst,
                    ignore=shutil.ignore_patterns("_lib", "__pycache__"))
    r = subprocess.run([sys.executable, "-c", "import fp32_sgemm_amd"], cwd=tmp_path,
                       capture_output=True, text=True)
    assert r.returncode != 0 and "ImportError" in r.stderr


# --- the benchmark's closed-form model against the pages' own figures -------
def test_flop_and_byte_counts_match_the_pages():
    import bench
    # "Writing a Fast Matmul in CUDA, Step by Step", Step 1: 2 x 4096^3 = 137.4
    # billion FLOPs; 3 x n^2 x 4 bytes = 201 MB; at most 683 FLOPs per byte.
    assert bench.gemm_flops(4096, 4096, 4096) == 137_438_953_472
    assert round(bench.gemm_min_bytes(4096, 4096, 4096, reads_c=False) / 1e6) == 201
    assert round(bench.arithmetic_intensity(4096, 4096, 4096, reads_c=False)) == 683
    # "How a Matmul Kernel Gets Fast", section 1 and 2: 2 x 4092^3 ~ 137 GFLOP;
    # read A, B and read+write C ~ 268 MB.
    assert round(bench.gemm_flops(4092, 4092, 4092) / 1e9) == 137
    assert round(bench.gemm_min_bytes(4092, 4092, 4092, reads_c=True) / 1e6) == 268
    # "Learn: Optimizing GEMM": the ideal intensity with 3n^2 traffic is n/6.
    assert abs(bench.arithmetic_intensity(4092, 4092, 4092, reads_c=False) - 4092 / 6) < 1e-9


def test_roofline_classification():
    import bench
    ridge = bench.PEAK_FP32_TFLOPS * 1e12 / (bench.PEAK_HBM_GBS * 1e9)
    assert 19 < ridge < 20
    assert bench.arithmetic_intensity(16, 4096, 4096, False) < ridge      # skinny: HBM-bound
    assert bench.arithmetic_intensity(4096, 4096, 4096, True) > ridge     # square: compute-bound
    assert bench.arithmetic_intensity(4096, 11008, 512, False) > ridge


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


# --- input generators ----------------------------------------------------------
def test_generators_are_deterministic_and_distinct():
    import workloads
    w = workloads.custom(37, 29, 41, "uniform", seed=3, beta=1.0, c0_dist="normal")
    A1, B1, C1 = workloads.make_inputs(w)
    A2, B2, C2 = workloads.make_inputs(w)
    assert np.array_equal(A1, A2) and np.array_equal(B1, B2) and np.array_equal(C1, C2)
    assert not np.array_equal(A1[:29, :29], B1[:29, :29])
    w2 = workloads.custom(37, 29, 41, "uniform", seed=4)
    assert not np.array_equal(workloads.make_inputs(w2)[0], A1)


def test_generator_distributions():
    import workloads
    u = workloads.draw((512, 512), "uniform", 1)
    assert u.dtype == np.float32 and u.min() >= -1.0 and u.max() < 1.0
    assert abs(float(u.mean())) < 0.01 and abs(float(u.std()) - (1 / 3) ** 0.5) < 0.01
    i = workloads.draw((512, 512), "int4", 2)
    assert set(np.unique(i).tolist()) == set(float(v) for v in range(-4, 5))
    n = workloads.draw((512, 512), "normal", 3)
    assert abs(float(n.mean())) < 0.01 and abs(float(n.std()) - 1.0) < 0.01
    p = workloads.draw((8, 5), "uniform", 4, pad_cols=3)
    assert p.shape == (8, 5) and p.strides[0] == 8 * 4


def test_named_workloads_match_the_configured_shapes():
    import workloads
    W = workloads.WORKLOADS
    assert (W["square4096_ab"].M, W["square4096_ab"].alpha, W["square4096_ab"].beta) == (4096, 1.5, -0.5)
    assert W["square4096_ab"].dist == "normal" and W["square4096_ab"].c0_dist == "normal"
    assert (W["skinny16x4096x4096"].M, W["skinny16x4096x4096"].N, W["skinny16x4096x4096"].K) == (16, 4096, 4096)
    assert (W["wide4096x11008x512"].N, W["wide4096x11008x512"].K) == (11008, 512)
    assert W["square128_int"].dist == "int4"
    assert workloads.HEADLINE == "square4096_ab"


def test_traffic_hash_ignores_comments_not_code():
    """bench.py reports the recorded HBM traffic only while the kernel source
    it was measured on is unchanged; comments and blank lines do not count."""
    import bench
    srcs = {rel: open(os.path.join(ROOT, rel), encoding="utf-8").read() for rel in bench.KERNEL_SOURCES}
    h = bench.kernel_source_hash(srcs)
    assert h == bench.kernel_source_hash()
    first = bench.KERNEL_SOURCES[0]
    commented = dict(srcs)
    commented[first] = "// a note\n\n" + srcs[first].replace("\n", "  // trailing note\n", 3)
    assert bench.kernel_source_hash(commented) == h
    changed = dict(srcs)
    changed[first] = srcs[first] + "\nint extra_symbol = 0;\n"
    assert bench.kernel_source_hash(changed) != h


def test_big_tiles_for_whole_filled_grids(sg):
    """Configuration 7 (256x256) is chosen for grids of 256x256 tiles that fill
    at least 95 % of their rounds of 256, and only where the plan would
    otherwise be the plain 128x128 grid; forced on a shape it cannot cover it
    refuses before any launch."""
    al = 0x100000
    plan = lambda ta, tb, M, N, K, lda, ldb: sg.sgemm_f32_ex_plan(ta, tb, M, N, K, 1.0, al, lda, al, ldb)
    for ta, tb in ((0, 0), (0, 1), (1, 0), (1, 1)):
        st, v, c, gm, s = plan(ta, tb, 4096, 4096, 4096, 4096, 4096)
        assert (st, v, c, s) == (0, sg.MFMA_TUNED, sg.CFG_256x256, 1), (ta, tb)
    for M, N, K in ((8192, 8192, 8192), (4096, 8192, 4096), (8192, 4096, 1024)):
        assert plan(0, 0, M, N, K, K, N)[2] == sg.CFG_256x256, (M, N, K)
    # Edge tiles are covered when M, N and K are multiples of 4 (4092^3: 16 x 16 tiles, the last 252 wide).
    assert plan(0, 0, 4092, 4092, 4092, 4092, 4092)[2] == sg.CFG_256x256
    assert plan(1, 1, 4092, 4092, 4092, 4092, 4092)[2] == sg.CFG_256x256
    # N of B as given, M of A transposed or K not a multiple of 4, misaligned,
    # too few or poorly filled rounds; M of A as given may be anything.
    assert plan(0, 0, 4096, 4094, 4096, 4096, 4096)[2] != sg.CFG_256x256
    assert plan(1, 0, 4094, 4096, 4096, 4096, 4096)[2] != sg.CFG_256x256
    assert plan(0, 0, 4094, 4096, 4096, 4096, 4096)[2] == sg.CFG_256x256
    assert plan(0, 0, 4096, 4096, 4098, 4098, 4096)[2] != sg.CFG_256x256
    assert sg.sgemm_f32_ex_plan(0, 0, 4096, 4096, 4100, 1.0, al + 4, 4100, al, 4096)[1] == sg.MFMA_SCALAR
    assert plan(0, 0, 2048, 2048, 2048, 2048, 2048)[2] != sg.CFG_256x256
    assert plan(0, 0, 6144, 6144, 2048, 2048, 6144)[2] != sg.CFG_256x256     # 576 tiles: 75 % of 3 rounds
    p = 0x100000
    for M, N, K in ((4096, 4094, 4096), (4096, 4098, 4096), (4096, 4096, 4098), (4096, 4096, 2)):
        assert sg.sgemm_f32_ex_config(7, 8, 1, 0, 0, M, N, K, 1.0, p, K + K % 4, p, N + N % 4, 0.0, p, N, 0) \
            == sg.ERR_NOT_APPLICABLE, (M, N, K)
    assert sg.sgemm_f32_ex_config(7, 8, 1, 0, 0, 512, 512, 64, 1.0, p + 4, 64, p, 512, 0.0, p, 512, 0) \
        == sg.ERR_NOT_APPLICABLE


def test_bench_median_of_last_three_quarters():
    """The pages' statistic: drop the first quarter of the launches, take the
    median of the rest (hand-worked: 8 launches, the first 2 dropped)."""
    import bench
    ms = [9.0, 8.0, 1.0, 5.0, 3.0, 4.0, 2.0, 6.0]
    # last three quarters: 1, 5, 3, 4, 2, 6 -> sorted 1 2 3 4 5 6 -> element 3 is 4
    assert bench.median_last_three_quarters(ms) == 4.0
    assert bench.median_last_three_quarters([7.0]) == 7.0


def test_bench_parity_leg_flags_a_wrong_element():
    """The benchmark's in-run parity check passes a result within the bound
    and fails one element moved past it, and reports the whole product."""
    import numpy as np

    import bench
    rng = np.random.default_rng(5)
    A = rng.standard_normal((33, 20)).astype(np.float32)
    B = rng.standard_normal((20, 17)).astype(np.float32)
    C0 = rng.standard_normal((33, 17)).astype(np.float32)
    good = (1.5 * (A.astype(np.float64) @ B.astype(np.float64)) - 0.5 * C0).astype(np.float32)
    parity, base = bench.parity_and_cpu_baseline(A, B, C0, 1.5, -0.5, good, False, None, 0.01)
    assert parity["ok"] and parity["elements"] == 33 * 17 and parity["n_bad"] == 0
    assert base["kind"] == "oracle" and base["cores"] >= 1
    bad = good.copy()
    bad[7, 3] += 1e-2
    parity, _ = bench.parity_and_cpu_baseline(A, B, C0, 1.5, -0.5, bad, False, None, 0.01)
    assert not parity["ok"] and parity["n_bad"] == 1 and parity["first_bad_index"] == [7, 3]
    Ai = rng.integers(-4, 5, (9, 11)).astype(np.float32)
    Bi = rng.integers(-4, 5, (11, 5)).astype(np.float32)
    exact = (Ai @ Bi).astype(np.float32)
    parity, _ = bench.parity_and_cpu_baseline(Ai, Bi, None, 1.0, 0.0, exact, True, None, 0.01)
    assert parity["ok"]
    exact[0, 0] = np.nextafter(exact[0, 0], np.float32(np.inf))
    parity, _ = bench.parity_and_cpu_baseline(Ai, Bi, None, 1.0, 0.0, exact, True, None, 0.01)
    assert not parity["ok"]
