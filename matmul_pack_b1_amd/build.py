"""Build libhyb.so (HIP, gfx950) in-tree with hipcc.

    python -m matmul_pack_b1_amd.build

Each source is compiled to an object in its own hipcc process (the kernel
files take minutes each, so they run in parallel), then the objects are
linked into one shared library.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libhyb.so")
SOURCES = ["hyb_api.cpp", "hyb_route.cpp", "hyb_pack.hip", "hyb_gemv.hip", "hyb_gemm.hip", "hyb_lowrank.hip"]
ARCH = os.environ.get("HYB_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # Packed-fp32 VALU forms stay disabled (they are not needed here).
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
    ]


def compile_cmd(src: str, obj: str) -> list[str]:
    return [hipcc()] + common_flags() + ["-c", "-o", obj, os.path.join(CSRC, src)]


def link_cmd(objs: list[str], out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out] + objs


def _run(cmd: list[str]) -> subprocess.CompletedProcess:
    return subprocess.run(cmd, capture_output=True, text=True)


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="hyb_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [compile_cmd(s, o) for s, o in zip(SOURCES, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        workers = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(_run, cmds))
        for src, res in zip(SOURCES, results):
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError(f"hipcc failed on {src} with exit code {res.returncode}")
        tmp = LIB_PATH + f".tmp{os.getpid()}"
        lc = link_cmd(objs, tmp)
        if verbose:
            print(" ".join(lc), flush=True)
        res = _run(lc)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"link failed with exit code {res.returncode}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
