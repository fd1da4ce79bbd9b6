"""Build the C consumer of the library (tests/c_abi/solve_poisson) with gcc, against
include/sla.h and the in-tree libsla.so (found at run time through a relative rpath)."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "differentiable_sparse_linear_spmv_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
EXE = os.path.join(HERE, "solve_poisson")


def build() -> str | None:
    if shutil.which("gcc") is None or not os.path.exists(os.path.join(PKG, "libsla.so")):
        return None
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), os.path.join(HERE, "solve_poisson.c"), "-o", EXE,
           "-L", PKG, "-l:libsla.so", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../differentiable_sparse_linear_spmv_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True)
    return EXE


if __name__ == "__main__":
    print(build())
