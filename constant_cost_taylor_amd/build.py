"""Build libsata.so (in-tree) for gfx950 with hipcc.

Usage:  python -m constant_cost_taylor_amd.build   (or call build_library()).
Every call recompiles.  Objects go to _build/ at the repository root; the
shared library lands next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libsata.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["sata_host.cpp", "sata_decode.hip", "sata_prefill.hip", "sata_prefill_b16.hip", "sata_softmax.hip"]
# The ceiling kernels (measurement tools) are a library of their own.
CEIL_SOURCES = ["sata_ceilings.hip"]
CEIL_OUT = os.path.join(PKG, "libsata_ceilings.so")

# Packed fp32 instructions are disabled for every HIP compile.
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the SATA library needs ROCm's hipcc")


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)


def build_library(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile and link libsata.so and libsata_ceilings.so; returns the first."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = list(extra or [])
    srcs = SOURCES + CEIL_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    _link(objs[:len(SOURCES)], OUT)
    _link(objs[len(SOURCES):], CEIL_OUT)
    if verbose:
        print(f"built {OUT}")
        print(f"built {CEIL_OUT}")
    return OUT


if __name__ == "__main__":
    build_library(verbose=True, extra=sys.argv[1:])
