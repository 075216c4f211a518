"""CPU sanitizer leg: the fp64 oracle and the C ABI's host-side argument validation, built
with AddressSanitizer and UndefinedBehaviorSanitizer, run the oracle's pins and the ABI's
error-path tests in child processes (the sanitizer runtime is preloaded there, since the
Python interpreter itself is not instrumented).  Only host code is instrumented: the
library's validation is linked with test stand-ins for its kernel launchers
(tests/san/launch_stubs.cpp), so nothing here needs a GPU."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_sscan_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_asan():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _clang_asan():
    base = os.path.join(ROCM, "lib", "llvm", "lib", "clang")
    if not os.path.isdir(base):
        return None
    for ver in sorted(os.listdir(base), reverse=True):
        p = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def _run_child(tests, env_extra, preload, tmp):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] + tests
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    log = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, log
    assert "ERROR: AddressSanitizer" not in log and "runtime error:" not in log, log
    return log


@pytest.mark.skipif(shutil.which("gcc") is None or _gcc_asan() is None, reason="gcc with libasan is needed")
def test_oracle_pins_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
                    "-fno-fast-math", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "sscan_oracle.c"), "-o", lib, "-lm"],
                   check=True)
    log = _run_child(["tests/test_oracle_pins.py", "tests/test_oracle_mamba_pins.py"],
                     {"SSCAN_ORACLE_LIBRARY": lib}, _gcc_asan(), tmp_path)
    assert "passed" in log


@pytest.mark.skipif(not os.path.exists(HIPCC) or _clang_asan() is None, reason="hipcc and clang's ASan runtime are needed")
def test_abi_validation_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    objs = []
    for src, lang in ((os.path.join(CSRC, "sscan_api.cpp"), "hip"), (os.path.join(ROOT, "tests", "san", "launch_stubs.cpp"), "hip")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        # sanitizers on the host pass only; the device pass (the scratch array) is built plain
        subprocess.run([HIPCC, "-x", lang, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                        "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                        "-c", src, "-o", obj], check=True, capture_output=True)
        objs.append(obj)
    lib = str(tmp_path / "libsscan_san.so")
    subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", lib] + objs, check=True,
                   capture_output=True)
    log = _run_child(["tests/test_abi.py", "tests/test_binding_host.py"], {"SSCAN_LIBRARY": lib}, _clang_asan(),
                     tmp_path)
    assert "passed" in log


CANARY = r"""
#include <stdlib.h>
int sscan_canary(int n) {  /* writes one element past a heap block of n ints */
  int* p = (int*)malloc(sizeof(int) * n);
  for (int i = 0; i <= n; ++i) p[i] = i;
  int s = p[0];
  free(p);
  return s;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None or _gcc_asan() is None, reason="gcc with libasan is needed")
def test_the_child_process_setup_reports_a_planted_overflow(tmp_path):
    """The harness itself: the same flags and preload catch a heap overflow planted in a
    throwaway C function, so a clean run of the tests above means something."""
    src = tmp_path / "canary.c"
    src.write_text(CANARY)
    lib = str(tmp_path / "libcanary.so")
    subprocess.run(["gcc", "-O0", "-g", "-fPIC", "-shared", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                    str(src), "-o", lib], check=True)
    env = dict(os.environ)
    env.update(SAN_ENV)
    env["LD_PRELOAD"] = _gcc_asan()
    code = f"import ctypes; ctypes.CDLL({lib!r}).sscan_canary(8)"
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
