"""Compile ``libfa06.so`` (the C-ABI library) for gfx950 with hipcc.

Run ``python -m flashattention_forward_06_amd.build`` or call :func:`build`.
The library is built in-tree next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

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


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with status {r.returncode}: {' '.join(cmd[-3:])}")


def build(verbose: bool = False, extra_flags=None, out: str | None = None) -> str:
    """Compile every source to an object in parallel (one hipcc per source),
    then link the shared library; the result replaces ``out`` atomically."""
    from concurrent.futures import ThreadPoolExecutor

    out = out or LIB_PATH
    tmp = out + ".tmp"
    objdir = tempfile.mkdtemp(prefix="fa06_build_")
    try:
        objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[HIPCC, *HIP_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", f"-I{CSRC}", "-c",
                 os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as pool:
            for f in [pool.submit(_run, c, verbose) for c in cmds]:
                f.result()
        _run([HIPCC, *HIP_FLAGS, *(extra_flags or []), "-shared", *objs, "-o", tmp], verbose)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
