"""Build the CPU oracle (test infrastructure) into oracle/libssm_oracle.so.

Plain gcc, -O2 with floating-point contraction off and no fast-math, so the
compiler neither fuses a multiply into an add nor reorders a sum.  OpenMP only
spreads independent (sequence, head) pairs over host threads.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ssm_oracle.c")
LIB = os.path.join(HERE, "libssm_oracle.so")

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC",
          "-shared", "-fopenmp", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB, extra=()) -> str:
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
