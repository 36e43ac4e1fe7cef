"""Build libfkmeans.so for gfx950 with hipcc, in-tree.

Usage: ``python -m exact_means_clustering_flashassign_amd.build`` (or the
``build()`` function). Always recompiles every source.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfkmeans.so")
SOURCES = ["norms.hip", "assign.hip", "assign_splitd.hip", "update.hip", "api.hip"]
# The contrast baselines (materialised-distance assign, scatter-atomic
# update) are a library of their own, linked against rocBLAS for the GEMM,
# so the Lloyd library itself depends on nothing but the HIP runtime.
BASELINE_LIB = os.path.join(HERE, "libfkbaseline.so")
BASELINE_SOURCES = ["baseline.hip"]
ROCM_LIB = "/opt/rocm/lib"
# Per-file flags. assign.hip: inputs are finite by contract, so fmaxf needs no
# NaN canonicalisation and the argmax max-tree lowers to plain v_max3_f32; its
# MFMA accumulators live in VGPRs, which the argmax reads without AGPR copies.
# assign_splitd.hip keeps the default (accumulators in AGPRs): its 256
# accumulator registers per lane would not fit the VGPR file.
FILE_FLAGS = {"assign.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libfkmeans")


def _compile(src: str, extra) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *FILE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out, libs=()) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, *libs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile and link libfkmeans.so and libfkbaseline.so; returns the former's path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = SOURCES + BASELINE_SOURCES
    jobs = min(len(srcs), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, list(extra_flags)), srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in BASELINE_SOURCES], BASELINE_LIB,
          [f"-L{ROCM_LIB}", f"-Wl,-rpath,{ROCM_LIB}", "-lrocblas"])
    if verbose:
        print(f"built {LIB} and {BASELINE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
