"""Build step for the HIP library: the translation units under csrc/ are
compiled in parallel with ``hipcc`` for gfx950 and linked into
``ssim_loss_amd/libssim_loss_amd.so``.

Packed-FP32 instructions are switched off (``-packed-fp32-ops``); the kernels
are written so that nothing depends on them.  Floating-point contraction is
limited to single expressions (``-ffp-contract=on``, not HIP's default of
fusing across statements): every fused multiply-add the arithmetic relies on
is written out, and a product stored to a variable must stay rounded -- the
forward's blurs by parts are exact on constant windows only if, say, a
squared difference is rounded before the difference from its neighbour is
taken.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
HEADERS = sorted(glob.glob(os.path.join(CSRC, "*.hpp")))
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libssim_loss_amd.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags(extra: list[str] | None = None) -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-ffp-contract=on",
            "-I", INCLUDE, "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            *(extra or [])]


def build(verbose: bool = False, extra: list[str] | None = None, build_dir: str = BUILD_DIR,
          lib_path: str = LIB_PATH) -> str:
    """Compile every csrc/*.hip and link lib_path.  `extra` compile flags go
    to every translation unit (a variant build, e.g. with host-side
    sanitizers, names its own build_dir and lib_path)."""
    os.makedirs(build_dir, exist_ok=True)
    cc = hipcc()

    def compile_one(src: str) -> str:
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        cmd = [cc, *compile_flags(extra), "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True))
