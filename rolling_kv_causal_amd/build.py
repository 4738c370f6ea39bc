"""Build libsdv2.so in-tree for gfx950 with hipcc (python -m rolling_kv_causal_amd.build)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import pathlib
import shutil
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = PKG / "_build"
LIB = PKG / "libsdv2.so"
SOURCES = ["sdv2.cpp", "k_append.hip", "k_attention.hip", "k_attention_w64.hip", "k_cache.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libsdv2.so)")


def _flags() -> list[str]:
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            # no packed-fp32 instructions in device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", str(ROOT / "include"), "-I", str(CSRC), "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> pathlib.Path:
    obj = BUILD / (src + ".o")
    cmd = [hipcc(), *_flags(), "-c", str(CSRC / src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n" + "\n".join(msgs))
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build(verbose: bool = True) -> pathlib.Path:
    """Compile every source for gfx950 and link libsdv2.so next to this file (always rebuilds)."""
    BUILD.mkdir(exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking libsdv2.so failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
