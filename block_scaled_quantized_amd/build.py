"""Build libmxgemm.so (HIP for gfx950) in-tree with hipcc.

Every source is compiled for gfx950 only, with packed-fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``). Objects go to ``_build/``; the shared
library lands next to this file. ``python -m block_scaled_quantized_amd.build`` runs it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import ctypes
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmxgemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "host_codec.cpp", "codec.hip", "mxgemm.hip", "mxgemm_ring.hip", "matvec.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]


# Per-source additions. matvec.hip: MFMA results go to ordinary VGPRs; its kernels scale every
# MFMA product on the vector ALU, and results left in accumulation registers would each need a
# v_accvgpr_read first (the GEMM kernels keep their accumulators in those registers and must not
# get this option).
EXTRA = {"matvec.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    # A kernel template that the host pass of hipcc fails to instantiate leaves an undefined device
    # stub behind without any diagnostic; linking a shared library lets that through, so resolve
    # every symbol now (no GPU is needed to load the library).
    try:
        ctypes.CDLL(tmp, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    except OSError as e:
        raise RuntimeError(f"built library does not load: {e}") from e
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
