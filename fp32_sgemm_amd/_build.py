"""Build step of the HIP library: compiles csrc/*.hip for gfx950 into _lib/.

The library is always rebuilt in place (a fresh shared object next to this
file), so the GPU tests, the smoke check and the benchmark load exactly the
code in the tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(HERE, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libsgemm_f32.so")
# A debug copy of the same library whose kernels fill their LDS with NaN before
# their first load (SGEMM_LDS_POISON): the tests run it to show that no stage is
# read before the loads that fill it have landed.  Never loaded by the package.
POISON_LIB_PATH = os.path.join(LIB_DIR, "libsgemm_f32_lds_poison.so")
OFFLOAD_ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed FP32 VALU instructions are switched off: the vector path is built from
# single v_fma_f32, and no packed form is ever emitted.
COMMON_FLAGS = [
    f"--offload-arch={OFFLOAD_ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, obj: str, remarks: bool, extra=()) -> str:
    cmd = [HIPCC, *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    if remarks:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{p.stderr}")
    keep = [ln for ln in p.stderr.splitlines()
            if "remark" in ln or ("error" in ln and "packed-fp32" not in ln)]
    return "\n".join(keep)


def build_library(jobs: int = 8, remarks: bool = True, poison: bool = False) -> str:
    """Compile every csrc/*.hip and link libsgemm_f32.so (with ``poison``, the
    LDS-poisoning debug copy instead); returns its path."""
    os.makedirs(LIB_DIR, exist_ok=True)
    lib_path = POISON_LIB_PATH if poison else LIB_PATH
    tag = ".poison" if poison else ""
    extra = ("-DSGEMM_LDS_POISON=1",) if poison else ()
    objs, reports = [], []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = {}
        for src in sources():
            obj = os.path.join(LIB_DIR, os.path.basename(src)[:-4] + tag + ".o")
            objs.append(obj)
            futs[ex.submit(_compile, src, obj, remarks and not poison, extra)] = src
        for f in cf.as_completed(futs):
            reports.append(f"== {os.path.basename(futs[f])}\n{f.result()}")
    tmp = lib_path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={OFFLOAD_ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr}")
    os.replace(tmp, lib_path)
    for o in objs:
        os.remove(o)
    if not poison:
        with open(os.path.join(LIB_DIR, "resource_usage.txt"), "w") as f:
            f.write("\n".join(sorted(reports)) + "\n")
    return lib_path


if __name__ == "__main__":
    print(build_library())
    print(build_library(poison=True))
