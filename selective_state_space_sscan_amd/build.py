"""Build libsscan.so for gfx950 with hipcc, in-tree.

    python -m selective_state_space_sscan_amd.build

Every HIP translation unit is compiled with packed-FP32 instruction selection
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass
warns that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsscan.so")
# microbenchmarks of the ceilings the kernels are measured against (bench.py --micro)
MICRO_SOURCES = ["micro.hip"]
MICRO_LIB = os.path.join(PKG, "libsscan_micro.so")

ARCH = os.environ.get("SSCAN_OFFLOAD_ARCH", "gfx950")
SOURCES = ["sscan_api.cpp", "fwd.hip", "fwd_mamba.hip", "fwd_sg.hip", "fwd_sg_mamba.hip", "bwd.hip", "bwd_mamba.hip",
           "bwd_hf.hip", "decode.hip"]


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsscan)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, verbose: bool) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + f".tmp{os.getpid()}"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every translation unit and link libsscan.so (and the microbenchmark
    library libsscan_micro.so) next to this file."""
    srcs = SOURCES + MICRO_SOURCES
    with cf.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], MICRO_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
