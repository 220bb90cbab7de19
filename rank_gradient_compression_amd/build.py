"""Builds the HIP library (libpowersgd.so) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIBNAME = "libpowersgd.so"
SOURCES = ["host.cpp", "kernels.hip", "noalloc.hip"]

# Packed fp32 instructions are switched off for every HIP translation unit.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def library_path() -> str:
    return os.path.join(LIBDIR, LIBNAME)


def build(verbose: bool = False, defines: dict | None = None, out: str | None = None) -> str:
    """Compiles the library. `defines` overrides the build-time tuning constants
    (PSGD_PASS1_ROWS, PSGD_PASS2_ROWS, PSGD_PASS3_ROWS, PSGD_TILES_PER_BUCKET); `out`
    writes the library elsewhere than the package's lib/ folder."""
    out = out or library_path()
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    macros = [f"-D{k}={v}" for k, v in sorted((defines or {}).items())]
    cmd = [hipcc(), *HIP_FLAGS, *macros, "-shared", "-I", os.path.join(ROOT, "include"), "-I",
           CSRC, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError(f"hipcc failed with exit code {proc.returncode}")
    if verbose and proc.stderr.strip():
        sys.stderr.write(proc.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
