"""Host code under AddressSanitizer + UndefinedBehaviorSanitizer (CPU only).

Two builds, each run by the existing CPU tests in a child process:

* the C-ABI library with its host code (argument validation, workspace
  arithmetic, strides and offsets; ``csrc/api.cpp``) compiled with
  ``-fsanitize=address,undefined`` for the host pass only -- the device code
  is not instrumented -- and linked with the ordinary kernel objects; the
  ABI validation tests then drive every entry point's error paths through
  it, with the clang ASan runtime preloaded into the interpreter;
* the fp64 oracle compiled by gcc with the same sanitizers, run by the
  oracle's pin and golden-value tests with gcc's ASan runtime preloaded.

Any sanitizer report aborts the child (``-fno-sanitize-recover=all``,
``halt_on_error``), which fails the test.  Leak checking is off: the
interpreter and the HIP runtime keep allocations until exit by design.
"""
import glob
import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
PKG = ROOT / "differential_attention_diffattn_amd"
SAN_FLAGS = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ASAN_OPTIONS = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
UBSAN_OPTIONS = "halt_on_error=1:print_stacktrace=1"


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _gcc_asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p) else None


def _run_child(env_extra, tests, tmp_path):
    env = dict(os.environ, ASAN_OPTIONS=ASAN_OPTIONS, UBSAN_OPTIONS=UBSAN_OPTIONS, **env_extra)
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-m", "not gpu", "-p", "no:cacheprovider", *tests]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    (tmp_path / "child.log").write_text(out)
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_abi_host_code_under_sanitizers(tmp_path):
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("no clang ASan runtime in this ROCm install")
    from differential_attention_diffattn_amd import build

    kernels = [s for s in build.SOURCES if s != "api.cpp"]
    objs = [build.BUILD_DIR / (s + ".o") for s in kernels]
    if not all(o.exists() for o in objs):
        build.build_library(verbose=False)
    host_san = [f for flag in SAN_FLAGS for f in ("-Xarch_host", flag)]
    api_obj = tmp_path / "api_san.o"
    subprocess.run([build.HIPCC, *build.FLAGS, *host_san, "-g", "-c", str(PKG / "csrc" / "api.cpp"),
                    "-o", str(api_obj)], check=True, capture_output=True)
    lib = tmp_path / "libdiffattn_san.so"
    subprocess.run([build.HIPCC, f"--offload-arch={build.ARCH}", "-shared", "-fPIC", "-shared-libasan",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    str(api_obj), *map(str, objs), "-o", str(lib)], check=True, capture_output=True)
    out = _run_child({"LD_PRELOAD": rt, "DIFFATTN_LIBRARY": str(lib)}, ["tests/test_abi_cpu.py"], tmp_path)
    assert " passed" in out


def test_oracle_under_sanitizers(tmp_path):
    rt = _gcc_asan_runtime()
    if rt is None:
        pytest.skip("gcc has no ASan runtime here")
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", *SAN_FLAGS,
                    str(ROOT / "oracle" / "diffattn_oracle.c"), "-o", str(lib), "-lm"],
                   check=True, capture_output=True)
    out = _run_child({"LD_PRELOAD": rt, "DIFFATTN_ORACLE_LIBRARY": str(lib)},
                     ["tests/test_oracle_pins.py", "tests/test_golden.py"], tmp_path)
    assert " passed" in out
