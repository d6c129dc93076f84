"""The C ABI's host code (argument checks, planning, routing:
hyb_api.cpp and hyb_route.cpp) built by the host compiler with the address
and undefined-behaviour sanitizers, with stand-in launchers
(tests/sanitize_launch_stub.cpp), and the CPU ABI tests run against that
build: every error path and the planning code run under the sanitizers."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "matmul_pack_b1_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _asan_runtime(gxx):
    out = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.slow
def test_abi_tests_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("needs g++ and the HIP headers")
    asan = _asan_runtime(gxx)
    if asan is None:
        pytest.skip("no libasan for this compiler")
    lib = str(tmp_path / "libhyb_sanitized.so")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           "-o", lib,
           os.path.join(CSRC, "hyb_api.cpp"), os.path.join(CSRC, "hyb_route.cpp"),
           os.path.join(ROOT, "tests", "sanitize_launch_stub.cpp"),
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ)
    env.update({
        "HYB_LIB": lib,
        "LD_PRELOAD": asan,
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    run = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q", "-x",
                          "-p", "no:cacheprovider", "-m", "not gpu"],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    tail = (run.stdout + run.stderr)[-4000:]
    assert run.returncode == 0, tail
    assert "passed" in run.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
