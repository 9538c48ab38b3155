"""Build libgemm_bf16.so in-tree from tiled_matmul_amd/csrc with hipcc for gfx950.

Every HIP source is compiled with the packed-fp32 instructions disabled (they are emitted by
hipcc -O3 from ordinary float code otherwise).  Objects go to tiled_matmul_amd/_build/.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgemm_bf16.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# Per-file compiler options.  The pipelined GEMM keeps MFMA fragments live across its K-block
# loop; LLVM's default scheduler then over-commits VGPRs and shuffles accumulators through
# AGPR copies, which the iterative ILP scheduler avoids.
FILE_FLAGS = {"gemm_pipe.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
              "gemm_ring.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}


def _compile(src: str, build_dir: str = BUILD, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-I", os.path.dirname(src),
           *[f"-D{d}" for d in defines], "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build_library(jobs: int | None = None, out: str = LIB, defines=(), csrc: str = CSRC) -> str:
    """Compile every csrc/*.hip and link libgemm_bf16.so (or ``out``).  Always recompiles.
    ``defines`` (NAME=VALUE strings) override the tile-shape macros of the kernels; ``csrc``
    selects another source directory with the same layout."""
    build_dir = BUILD if out == LIB else os.path.join(os.path.dirname(os.path.abspath(out)), "_build")
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(csrc, "*.hip")))
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, defines), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


CEILING_SRC = os.path.join(PKG, "ceiling", "ceiling.hip")
CEILING_LIB = os.path.join(PKG, "ceiling", "libtmm_ceiling.so")


def build_ceiling() -> str:
    """Compile libtmm_ceiling.so (the measurement kernels bench.py runs beside the GEMV)."""
    tmp = CEILING_LIB + ".tmp"
    cmd = [HIPCC, *CFLAGS, "-shared", CEILING_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {CEILING_SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, CEILING_LIB)
    return CEILING_LIB


if __name__ == "__main__":
    print(build_library())
