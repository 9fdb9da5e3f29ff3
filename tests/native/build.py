"""Build tests/native/abi_consumer: a plain C program (gcc, HIP runtime API
only) linked against libarrms.so and the CPU oracle, run by
tests/test_native_consumer_gpu.py. Call after both libraries are built."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
BIN = os.path.join(HERE, "abi_consumer")


def build() -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROOT}/include", f"-I{ROCM}/include", os.path.join(HERE, "abi_consumer.c"), "-o", BIN,
           f"-L{ROOT}/all_reduce_residual_rank_amd", "-larrms", f"-L{ROOT}/oracle", "-loracle",
           f"-L{ROCM}/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../all_reduce_residual_rank_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
           f"-Wl,-rpath,{ROCM}/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed on abi_consumer.c:\n{r.stderr}")
    return BIN


if __name__ == "__main__":
    print(build())
