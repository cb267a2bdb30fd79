"""Compile ``libfa06.so`` (the C-ABI library) for gfx950 with hipcc.

Run ``python -m flashattention_forward_06_amd.build`` or call :func:`build`.
The library is built in-tree next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libfa06.so")
SOURCES = ["fa_api.cpp", "fa_fwd_kernel.hip", "fa_bwd_kernel.hip", "fa_fwd_mxfp8.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions stay off: scalar float code only.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False, extra_flags=None, out: str | None = None) -> str:
    out = out or LIB_PATH
    tmp = out + ".tmp"
    cmd = [HIPCC, *HIP_FLAGS, *(extra_flags or []), "-shared", f"-I{INCLUDE}", f"-I{CSRC}",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with status {r.returncode}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
