"""Build step for the CPU oracle: ``gcc -O2 -fopenmp -shared``.

Test infrastructure only (see ``ssim_oracle.c``).  No -ffast-math: the oracle's
fp64 arithmetic must follow IEEE rounding so that its pins are meaningful.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ssim_oracle.c")
LIB_PATH = os.path.join(HERE, "libssim_oracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
