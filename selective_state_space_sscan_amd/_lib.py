"""ctypes declarations for libsscan's C ABI (include/sscan.h).

Loading the library touches no GPU.  If libsscan.so has not been built the
loader raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
# SSCAN_LIBRARY names another build of the same library (the host-sanitizer test loads one
# whose host code is instrumented); by default the in-tree build.
LIB_PATH = os.environ.get("SSCAN_LIBRARY") or os.path.join(PKG, "libsscan.so")

SSCAN_F32 = 0
SSCAN_BF16 = 1

STATUS_NAMES = {
    0: "SSCAN_OK",
    1: "SSCAN_ERR_NULL",
    2: "SSCAN_ERR_SHAPE",
    3: "SSCAN_ERR_DTYPE",
    4: "SSCAN_ERR_UNSUPPORTED",
    5: "SSCAN_ERR_ALIGN",
    6: "SSCAN_ERR_WORKSPACE",
    7: "SSCAN_ERR_HIP",
}

# Every function include/sscan.h declares.
EXPORTED = ("sscan_fwd", "sscan_fwd_workspace", "sscan_fwd_noalloc", "sscan_bwd", "sscan_bwd_workspace", "sscan_mamba_fwd",
            "sscan_mamba_bwd", "sscan_mamba_bwd_workspace", "sscan_fwd_ckpt", "sscan_bwd_ckpt",
            "sscan_bwd_ckpt_workspace", "sscan_decode", "sscan_plan_select", "sscan_status_str",
            "sscan_last_error", "sscan_version")
SSCAN_CKPT_STEPS = 32
SSCAN_NOALLOC_SCRATCH_BYTES = 32 << 20
SSCAN_WRAP_NONE = 0
SSCAN_WRAP_MAMBA = 1
SSCAN_LAYOUT_AUTO = 0
SSCAN_LAYOUT_LANES = 1
SSCAN_LAYOUT_STATE_GROUPS = 2


class sscan_desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("D", ctypes.c_int64), ("DS", ctypes.c_int64),
                ("io", ctypes.c_int32), ("reserved", ctypes.c_int32), ("x_bstride", ctypes.c_int64),
                ("bc_bstride", ctypes.c_int64), ("y_bstride", ctypes.c_int64)]


class sscan_plan(ctypes.Structure):
    _fields_ = [("lanes", ctypes.c_int32), ("chunks", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 5)]


class SScanError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


_lock = threading.Lock()
_lib = None


def load() -> ctypes.CDLL:
    """Load libsscan.so (built in-tree by ``selective_state_space_sscan_amd.build``)."""
    global _lib
    if _lib is not None:  # loaded: no lock needed to read the reference
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m selective_state_space_sscan_amd.build` "
                               "(the HIP library is required; there is no fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        pdesc, pplan = ctypes.POINTER(sscan_desc), ctypes.POINTER(sscan_plan)
        lib.sscan_fwd.argtypes = [pdesc, pplan] + [vp] * 9 + [vp, sz, vp]
        lib.sscan_fwd.restype = i32
        lib.sscan_fwd_noalloc.argtypes = [pdesc, pplan] + [vp] * 9 + [vp]
        lib.sscan_fwd_noalloc.restype = i32
        lib.sscan_fwd_workspace.argtypes = [pdesc, pplan, ctypes.POINTER(sz)]
        lib.sscan_fwd_workspace.restype = i32
        lib.sscan_bwd.argtypes = [pdesc, pplan] + [vp] * 15 + [vp, sz, vp]
        lib.sscan_bwd.restype = i32
        lib.sscan_bwd_workspace.argtypes = [pdesc, pplan, ctypes.POINTER(sz)]
        lib.sscan_bwd_workspace.restype = i32
        lib.sscan_mamba_fwd.argtypes = [pdesc, pplan] + [vp] * 10 + [vp, sz, vp]
        lib.sscan_mamba_fwd.restype = i32
        lib.sscan_mamba_bwd.argtypes = [pdesc, pplan] + [vp] * 17 + [vp, sz, vp]
        lib.sscan_mamba_bwd.restype = i32
        lib.sscan_mamba_bwd_workspace.argtypes = [pdesc, pplan, ctypes.POINTER(sz)]
        lib.sscan_mamba_bwd_workspace.restype = i32
        lib.sscan_fwd_ckpt.argtypes = [pdesc, pplan, i32] + [vp] * 10 + [vp, sz, vp]
        lib.sscan_fwd_ckpt.restype = i32
        lib.sscan_bwd_ckpt.argtypes = [pdesc, pplan, i32] + [vp] * 16 + [vp, sz, vp]
        lib.sscan_bwd_ckpt.restype = i32
        lib.sscan_bwd_ckpt_workspace.argtypes = [pdesc, pplan, i32, ctypes.POINTER(sz)]
        lib.sscan_bwd_ckpt_workspace.restype = i32
        lib.sscan_decode.argtypes = [pdesc] + [vp] * 8 + [vp]
        lib.sscan_decode.restype = i32
        lib.sscan_plan_select.argtypes = [pdesc, i32, pplan]
        lib.sscan_plan_select.restype = i32
        lib.sscan_status_str.argtypes = [i32]
        lib.sscan_status_str.restype = ctypes.c_char_p
        lib.sscan_last_error.argtypes = []
        lib.sscan_last_error.restype = ctypes.c_char_p
        lib.sscan_version.argtypes = []
        lib.sscan_version.restype = i32
        _lib = lib
        return lib


def check(status: int) -> None:
    if status != 0:
        msg = load().sscan_last_error().decode(errors="replace")
        raise SScanError(status, msg)
