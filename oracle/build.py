"""Builds the oracle's C sources into oracle/liboracle.so with gcc.

Test infrastructure: the oracle is compiled so tests and the CPU baseline can
call it; the product library never links it.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SOURCES = ["fp16.c", "formats.c", "ops.c", "model.c"]


def build_oracle(verbose: bool = False) -> str:
    # -ffp-contract=off: every operation rounds exactly as written.
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-pthread", "-Wall", "-Wextra", "-Wno-unused-parameter", "-D_GNU_SOURCE",
           "-o", LIB_PATH + ".tmp"] + [os.path.join(HERE, s) for s in SOURCES] + ["-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_oracle(verbose=True))
