"""Compile gemm_from_c.c, the plain C caller of the C ABI, with gcc (C99,
warnings as errors) against include/dense_gemm.h, linked to the in-tree
libdense_gemm_amd.so and the HIP runtime.

    python tests/c_abi/build.py
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "gemm_from_c.c")
EXE = os.path.join(HERE, "gemm_from_c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    pkg = os.path.join(ROOT, "dense_gemm_amd")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-isystem", os.path.join(ROCM, "include"), SRC, "-o", EXE + ".tmp",
           "-L", pkg, "-ldense_gemm_amd", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../dense_gemm_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build())
