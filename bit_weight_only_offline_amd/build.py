"""Build the HIP library libqlinear.so in-tree for gfx950 with hipcc.

Each source compiles to an object under _build/ in parallel, then one link step
produces bit_weight_only_offline_amd/libqlinear.so.  Run as a module or call build().
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqlinear.so")

SOURCES = [   # slowest first, so the parallel build starts them first
    "ql_gemm_int4_zp.hip",
    "ql_gemm_int4.hip",
    "ql_gemm_int8.hip",
    "ql_gemm_cb4.hip",
    "ql_gemm_mxfp4.hip",
    "ql_gemm_a8.hip",
    "ql_api.hip",
    "ql_pack.hip",
    "ql_misc.hip",
    "ql_quant.hip",
    "ql_lora.hip",
]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Wno-unused-function",
    # no packed-fp32 (v_pk_*_f32) instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


# Per-source flags.  The INT8-compute kernel keeps its matrix-core accumulators in
# ordinary VGPRs (no copies to and from AGPRs around the MFMAs): measured 52.5 against
# 66.8 us for W8A8 at 3072 x 3072, M = 2048, and 23.8 against 25.8 us at M = 256.  The
# bf16 tile kernels measured the same or slower with it, so they keep the default.
SOURCE_FLAGS = {
    "ql_gemm_a8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-8000:]}")
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    """Compile every source and link libqlinear.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-8000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
