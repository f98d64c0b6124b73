"""Compile the CPU oracle (plain C) into oracle/libcfz_oracle.so with gcc.

Strict IEEE semantics: no fast-math and no floating-point contraction, so that
the only fused multiply-adds are the explicit fmaf calls of the definitions.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cfz_oracle.c")
LIB = os.path.join(HERE, "libcfz_oracle.so")
# The same source with OpenMP: its independent outer loops (groups, rows, columns)
# split among threads, each output computed by one thread in the serial build's
# order, so the two libraries give identical bits.
LIB_OMP = os.path.join(HERE, "libcfz_oracle_omp.so")

CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
          "-fno-strict-aliasing", "-Wall", "-Wextra", "-Wno-unused-parameter",
          "-Wno-unknown-pragmas"]


def _build_one(out, extra, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *extra, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    _build_one(LIB, [], verbose)
    _build_one(LIB_OMP, ["-fopenmp"], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
