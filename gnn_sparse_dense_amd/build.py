"""Build libgnn_spmm.so (HIP, gfx950) in-tree with hipcc.

Each translation unit under csrc/ is compiled separately (in parallel) and the
objects are linked into gnn_sparse_dense_amd/libgnn_spmm.so next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgnn_spmm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = [
    "api.cpp",
    "alloc.cpp",
    "plan_kernels.hip",
    "combine.hip",
    "row_kernels_v1.hip",
    "row_kernels_v2.hip",
    "row_kernels_v4.hip",
    "window_kernels.hip",
    "transform.hip",
    "mfma_tile.hip",
    "features.hip",
    "pair_kernel.hip",
    "reorder.hip",
    "merge_kernel.hip",
    "split_fused.hip",
]

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-result",
    # no packed fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division for the mean (also hipcc's default; stated explicitly)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _compile(src: str) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") or src.endswith(".cpp") else []
    cmd = [HIPCC, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return out


def build(verbose: bool = True, jobs: int = 8) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
