"""Host-only sanitizer run: the C-ABI shim's validation path and the fp64
oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (g++ and
gcc; the kernel launchers are host stubs, so nothing runs on a GPU).

The driver (tests/sanitize/sanitize_driver.cpp) calls every entry point of
include/fa06.h with each kind of argument it must reject and once with valid
arguments, and runs the oracle's entry points on small and degenerate inputs;
any out-of-bounds access, use after free, leak or undefined behaviour aborts
it with a sanitizer report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "flashattention_forward_06_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def test_validation_and_oracle_under_sanitizers(tmp_path):
    if shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers are missing")
    out = str(tmp_path)
    cxx = ["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{CSRC}",
           "-Wall", *SAN]
    objs = []
    for src in (os.path.join(CSRC, "fa_api.cpp"), os.path.join(HERE, "stub_launch.cpp"),
                os.path.join(HERE, "sanitize_driver.cpp")):
        obj = os.path.join(out, os.path.basename(src) + ".o")
        subprocess.run([*cxx, "-c", src, "-o", obj], check=True)
        objs.append(obj)
    obj = os.path.join(out, "fa_oracle.o")
    subprocess.run(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", "-Wall", *SAN, "-c",
                    os.path.join(ROOT, "oracle", "fa_oracle.c"), "-o", obj], check=True)
    objs.append(obj)
    exe = os.path.join(out, "sanitize_driver")
    subprocess.run(["g++", *SAN, *objs, "-fopenmp", f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib",
                    "-lm", "-o", exe], check=True)
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="abort_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.startswith("SANITIZE_OK"), r.stdout
