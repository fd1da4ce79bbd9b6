"""Compile the CPU oracle (test infrastructure) into oracle/libsla_oracle.so.

Plain gcc, no contraction, so every product is rounded before it is summed.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sla_oracle.c")
LIB = os.path.join(HERE, "libsla_oracle.so")


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    # -fopenmp serves orc_cg_timing and orc_bicgstab_timing (the CPU baseline's timing
    # modes) only; the parity functions have no OpenMP pragmas and run sequentially
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c99", "-Wall", "-fopenmp",
           "-shared", "-fPIC", SRC, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True))
    sys.exit(0)
