"""Build libarrms.so (gfx950) in-tree: ``python -m all_reduce_residual_rank_amd.build``.

Compiles the three per-dtype kernel translation units and the C-ABI host code
with hipcc in parallel, then links the shared library next to this file.
Always recompiles. Object files go to ``_build/`` at the repository root.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libarrms.so")

SOURCES = ["kern_bf16_t.hip", "kern_bf16_fp8.hip", "kern_bf16_fp8t.hip", "kern_fp16_t.hip",
           "kern_fp16_fp8.hip", "kern_fp16_fp8t.hip", "kern_fp32_t.hip", "kern_bf16_fp8g.hip",
           "kern_bf16_mx4.hip", "kern_fp16_fp8g.hip", "kern_fp16_mx4.hip", "api.cpp", "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# -packed-fp32-ops: keep the compiler from forming packed fp32 arithmetic;
# -fno-gpu-flush-denormals-to-zero: IEEE subnormals in fp32 conversions.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fno-gpu-flush-denormals-to-zero", f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".", "_") + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
