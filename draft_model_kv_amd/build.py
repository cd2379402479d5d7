"""Build the HIP library libringkv.so in-tree for gfx950 (MI355X).

Run ``python draft_model_kv_amd/build.py`` (it does not import the package, so a
stale library never blocks a rebuild) or call ``build()``.  The library
is written next to this file, where ``draft_model_kv_amd.ring`` loads it.
The same sources are also built with per-wave timestamps into
libringkv_stamps.so, a profiling build that ``draft_model_kv_amd.ring``
loads instead when RINGKV_LIB=stamps.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libringkv.so")
# the same sources with per-wave timestamps (profiling only: ring_profile_stamps)
LIB_STAMPS = os.path.join(PKG, "libringkv_stamps.so")
SOURCES = ["ring_runtime.cpp", "ring_kernels.hip", "ring_floor.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libringkv.so)")


def command(out: str, stamps: bool = False) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    ] + (["-DRING_WAVE_STAMPS"] if stamps else []) + [
        "-Wall", "-Wno-unused-function",
        # packed FP32 instructions stay off: plain scalar FP32 code only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
        "-o", out,
    ] + [os.path.join(CSRC, s) for s in SOURCES]


def build_one(lib: str, stamps: bool, verbose: bool) -> subprocess.Popen:
    cmd = command(lib + ".tmp", stamps)
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def build(verbose: bool = False) -> str:
    """Compile both libraries (in parallel); returns the product library's path."""
    jobs = [(lib, build_one(lib, stamps, verbose))
            for lib, stamps in ((LIB, False), (LIB_STAMPS, True))]
    noise = "is not a recognized feature for this target"
    failed = []
    for lib, p in jobs:
        _, stderr = p.communicate()
        err = "\n".join(l for l in stderr.splitlines() if noise not in l)
        if p.returncode != 0:
            failed.append(f"{os.path.basename(lib)}: hipcc failed ({p.returncode}):\n{err}")
            continue
        if verbose and err.strip():
            print(err, file=sys.stderr)
        os.replace(lib + ".tmp", lib)
    if failed:
        raise RuntimeError("\n".join(failed))
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
