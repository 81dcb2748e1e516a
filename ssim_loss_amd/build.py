"""Build step for the HIP library: one ``hipcc`` call producing
``ssim_loss_amd/libssim_loss_amd.so`` for gfx950.

Packed-FP32 instructions are switched off (``-packed-fp32-ops``); the kernels
are written so that nothing depends on them.
"""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "ssim_kernels.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libssim_loss_amd.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_cmd(out: str, extra: list[str] | None = None) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-I", INCLUDE,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            *(extra or []), "-o", out, SRC]


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = compile_cmd(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
