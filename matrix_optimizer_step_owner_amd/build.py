"""Build the HIP library ``libmfsdp.so`` in-tree for gfx950.

Usage:  python -m matrix_optimizer_step_owner_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_PATH = os.path.join(PKG_DIR, "libmfsdp.so")
SOURCES = [os.path.join(PKG_DIR, "csrc", "mfsdp.hip")]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, arch: str = "gfx950") -> str:
    """Compile the library (always recompiles) and return its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={arch}", "-O3", "-std=c++17", "-fPIC",
           "-shared",
           # no packed-fp32 VALU instructions anywhere in device code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"),
           "-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
