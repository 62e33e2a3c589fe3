"""Build libdiffattn.so in-tree with hipcc for gfx950.

    python -m differential_attention_diffattn_amd.build

Every translation unit is compiled with packed-fp32 instruction generation
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host
pass warns that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
OUT = PKG / "libdiffattn.so"
BUILD_DIR = PKG.parent / "_build"
SOURCES = ["api.cpp", "prefill_bf16.hip", "v1_fp32.hip", "decode_bf16.hip", "backward_bf16.hip", "prologue_bf16.hip"]
ARCH = os.environ.get("DIFFATTN_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]
# Per-source additions (none at present: every kernel's launch bounds allow
# at least two waves per SIMD, so the compiler keeps MFMA results in VGPRs).
EXTRA: dict[str, list[str]] = {}


def _compile(src: str) -> Path:
    obj = BUILD_DIR / (Path(src).name + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", str(CSRC / src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build_library(verbose: bool = True) -> Path:
    """Compile every HIP/C++ source and link libdiffattn.so next to this file."""
    BUILD_DIR.mkdir(exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT.with_suffix(f".so.tmp{os.getpid()}")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT} ({OUT.stat().st_size} bytes)")
    return OUT


if __name__ == "__main__":
    build_library()
