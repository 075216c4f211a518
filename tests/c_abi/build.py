"""Compile the plain-C consumer of libsscan (tests/c_abi/dyadic.c) with gcc, linked
against the in-tree libsscan.so (found at run time through its rpath)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "selective_state_space_sscan_amd")
EXE = os.path.join(HERE, "dyadic")


def build() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(rocm, "include"), os.path.join(HERE, "dyadic.c"), "-o", EXE,
           "-L", PKG, "-l:libsscan.so", "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../selective_state_space_sscan_amd", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    subprocess.run(cmd, check=True)
    return EXE


if __name__ == "__main__":
    print(build())
