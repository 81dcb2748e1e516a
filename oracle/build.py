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


def build(verbose: bool = False, cc: str = "gcc", extra: list[str] | None = None,
          lib_path: str = LIB_PATH) -> str:
    """Compile the oracle into lib_path.  A variant build (another compiler,
    sanitizer flags in `extra`) names its own lib_path."""
    tmp = lib_path + ".tmp"
    cmd = [cc, "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           *(extra or []), "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True))
