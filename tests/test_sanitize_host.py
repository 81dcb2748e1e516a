"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

The oracle (C) and the C-ABI library's host side (argument checks, shape and
size arithmetic, the workspace and scratch bookkeeping) are rebuilt with
clang's ASan + UBSan -- the HIP translation units with the sanitizers on the
host pass only; device code is built as usual -- and the oracle pins and the
host ABI tests run again in a child process that preloads the ASan runtime and
loads those builds (SSIM_ORACLE_LIB, SSIM_LOSS_AMD_LIB).  Any report ends the
child with an error.  Skipped where the toolchain or the runtime is absent.
"""
import importlib
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
FILES = ["tests/test_oracle_pins.py", "tests/test_oracle_pins3d.py", "tests/test_abi_host.py"]
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _asan_runtime():
    if not os.path.exists(CLANG):
        return None
    out = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True).stdout.strip()
    if os.path.isabs(out) and os.path.exists(out):
        return out
    rt = subprocess.run([CLANG, "--print-runtime-dir"], capture_output=True, text=True).stdout
    for name in ("libclang_rt.asan-x86_64.so", "libclang_rt.asan.so"):
        p = os.path.join(rt.strip(), name)
        if os.path.exists(p):
            return p
    return None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc is not installed")
    sys.path.insert(0, ROOT)
    # the modules, not the packages' build() functions of the same name
    ob = importlib.import_module("oracle.build")
    sb = importlib.import_module("ssim_loss_amd.build")

    d = tmp_path_factory.mktemp("sanitize")
    san = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined"]
    oracle_lib = ob.build(cc=CLANG, extra=[*san, "-Wl,-rpath,/opt/rocm/llvm/lib"],
                          lib_path=str(d / "liboracle_san.so"))
    host_only = ["-g", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-fsanitize=address,undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined"]
    hip_lib = sb.build(extra=host_only, build_dir=str(d / "obj"),
                       lib_path=str(d / "libssim_loss_amd_san.so"))
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, SSIM_ORACLE_LIB=oracle_lib, SSIM_LOSS_AMD_LIB=hip_lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               PYTHONDONTWRITEBYTECODE="1")
    return {"runtime": runtime, "oracle": oracle_lib, "hip": hip_lib, "env": env, "dir": d}


def _run(cmd, env, timeout=900):
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


def test_sanitizer_catches_a_heap_overflow(sanitized, tmp_path):
    """The runtime and options in use do report: a C program that reads one
    element past a heap array fails with a heap-buffer-overflow report."""
    src = tmp_path / "overflow.c"
    src.write_text("#include <stdlib.h>\n"
                   "int main(int c, char** v) { (void)v; int* a = malloc(4 * sizeof(int));\n"
                   "  for (int i = 0; i < 4; ++i) a[i] = i;\n"
                   "  int s = a[c + 3]; free(a); return s == 12345; }\n")
    exe = tmp_path / "overflow"
    subprocess.run([CLANG, "-g", "-fsanitize=address", "-o", str(exe), str(src)], check=True)
    env = {k: v for k, v in sanitized["env"].items() if k != "LD_PRELOAD"}
    r = subprocess.run([str(exe)], env=env, capture_output=True, text=True, timeout=60)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]


def test_sanitized_builds_are_the_ones_loaded(sanitized):
    code = ("import oracle, ssim_loss_amd as S; oracle._load(); S.lib(); "
            "print(open('/proc/self/maps').read())")
    r = _run([sys.executable, "-c", code], sanitized["env"], timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    for key in ("runtime", "oracle", "hip"):
        assert sanitized[key] in r.stdout, f"{sanitized[key]} is not mapped"


def test_oracle_pins_and_host_abi_under_asan_ubsan(sanitized):
    r = _run([sys.executable, "-m", "pytest", *FILES, "-q", "-x", "-m", "not gpu",
              "-p", "no:cacheprovider"], sanitized["env"])
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    for rep in REPORTS:
        assert rep not in out, out[-6000:]
    assert " passed" in r.stdout
