"""Selective diagonal state-space scan for AMD Instinct MI355X (gfx950).

    h_t = exp(delta_t * A) * h_{t-1} + delta_t * b_t * x_t,    y_t = <h_t, c_t>

(the "pssa-100m/pssa_kernels.py" page, module docstring).  The compute lives in
libsscan.so, hand-written HIP kernels behind a C ABI (include/sscan.h); this
package is its Python binding.  Build it with
``python -m selective_state_space_sscan_amd.build``.
"""
from .api import (MambaScan, Plan, SelectiveScan, SScanError, mamba_scan, selective_scan, sscan_bwd,
                  sscan_bwd_ckpt, sscan_bwd_workspace, sscan_decode, sscan_fwd, sscan_fwd_ckpt,
                  sscan_fwd_noalloc, sscan_fwd_workspace, sscan_mamba_bwd,
                  sscan_mamba_bwd_workspace, sscan_mamba_fwd, sscan_plan_select, sscan_version)

__all__ = ["MambaScan", "Plan", "SelectiveScan", "SScanError", "mamba_scan", "selective_scan", "sscan_bwd",
           "sscan_bwd_ckpt", "sscan_fwd_ckpt", "sscan_bwd_workspace", "sscan_decode", "sscan_fwd", "sscan_fwd_noalloc",
           "sscan_fwd_workspace", "sscan_mamba_bwd",
           "sscan_mamba_bwd_workspace", "sscan_mamba_fwd", "sscan_plan_select", "sscan_version"]
