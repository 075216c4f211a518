"""Python entry points of libsscan, named after the C ABI (include/sscan.h).

These functions only marshal arguments: they check tensor placement and
layout, let torch allocate outputs and workspace on the caller's device, and
call the C library on torch's current HIP stream.  Every step of the scan
runs in libsscan's gfx950 kernels.  Calls are asynchronous like any torch op.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import SScanError, sscan_desc, sscan_plan

__all__ = ["sscan_fwd", "sscan_fwd_noalloc", "sscan_bwd", "sscan_mamba_fwd", "sscan_mamba_bwd", "sscan_fwd_ckpt", "sscan_bwd_ckpt",
           "sscan_decode", "sscan_fwd_workspace",
           "sscan_bwd_workspace", "sscan_mamba_bwd_workspace", "sscan_plan_select", "sscan_version",
           "SelectiveScan", "selective_scan", "MambaScan", "mamba_scan", "SScanError", "Plan"]

_IO = {torch.float32: _lib.SSCAN_F32, torch.bfloat16: _lib.SSCAN_BF16}


class Plan:
    """Launch plan override: ``lanes`` per channel, T-``chunks`` and the forward's ``layout``
    (``"lanes"`` or ``"state_groups"``); 0 / None = the library's choice."""

    _LAYOUTS = {None: 0, "lanes": 1, "state_groups": 2}

    def __init__(self, lanes: int = 0, chunks: int = 0, layout: Optional[str] = None):
        if layout not in self._LAYOUTS:
            raise ValueError(f"layout must be one of {list(self._LAYOUTS)}, got {layout!r}")
        self.lanes = int(lanes)
        self.chunks = int(chunks)
        self.layout = layout

    def _c(self) -> sscan_plan:
        p = sscan_plan()
        p.lanes = self.lanes
        p.chunks = self.chunks
        p.layout = self._LAYOUTS[self.layout]
        return p

    def __repr__(self):
        return f"Plan(lanes={self.lanes}, chunks={self.chunks}, layout={self.layout!r})"


def _plan_ptr(plan: Optional[Plan]):
    if plan is None:
        return None, None
    c = plan._c()
    return c, ctypes.byref(c)


# The entry points' pointer arguments are declared c_void_p, so plain integers (and None
# for NULL) pass straight through ctypes.
def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: torch.device):
    """torch's current HIP stream on ``device``, as the integer handle the C ABI takes."""
    if _raw_stream is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _call(device: torch.device, fn, *args):
    """``fn(*args)`` with ``device`` current (the library launches on, and plans for, the
    current device); no device switch when it already is."""
    if device.index == torch.cuda.current_device():
        return fn(*args)
    with torch.cuda.device(device):
        return fn(*args)


_ws_cache = {}


def _ws_bytes(device: torch.device, kind: str, query, d: sscan_desc, plan: Optional[Plan], pp, *extra) -> int:
    """Workspace bytes of an entry point for (desc, plan), asked of the library once per
    shape, layout, plan and device (the answer depends on nothing else)."""
    key = (kind, device.index, d.B, d.T, d.D, d.DS, d.io, d.x_bstride, d.bc_bstride, d.y_bstride,
           None if plan is None else (plan.lanes, plan.chunks, plan.layout)) + extra
    n = _ws_cache.get(key)
    if n is None:
        nws = ctypes.c_size_t(0)
        _lib.check(_call(device, query, ctypes.byref(d), pp, *extra, ctypes.byref(nws)))
        if len(_ws_cache) >= 4096:  # many distinct shapes (e.g. a varying T): start over
            _ws_cache.clear()
        n = _ws_cache[key] = int(nws.value)
    return n


def _batch_stride(t: torch.Tensor, name: str) -> int:
    """Batch stride of a (B, R, C) tensor whose trailing (R, C) block is contiguous and
    whose batch rows do not overlap.  A tensor broadcast over the batch dimension (stride
    0, e.g. from ``expand``) is rejected: the C ABI reads a batch stride of 0 as R*C."""
    shape = t.shape
    if len(shape) != 3:
        raise ValueError(f"{name} must be 3-D, got shape {tuple(shape)}")
    B, R, C = shape
    s0, s1, s2 = t.stride()
    if C > 1 and s2 != 1 or R > 1 and s1 != C:
        raise ValueError(f"{name}: the last two dimensions must be contiguous")
    if B > 1 and s0 < R * C:
        raise ValueError(f"{name}: batch rows overlap (batch stride {s0} < {R * C})")
    return s0 if B > 1 else R * C


def _rows_view(t: torch.Tensor, name: str) -> Tuple[torch.Tensor, int]:
    try:
        return t, _batch_stride(t, name)
    except ValueError:
        t = t.contiguous()
        return t, _batch_stride(t, name)


def _same_stride(ts, names):
    """Bring tensors that must share one batch stride to a common layout."""
    try:  # the common case: every tensor already has the row layout, with one stride
        strides = [_batch_stride(t, n) for t, n in zip(ts, names)]
        if all(s_ == strides[0] for s_ in strides):
            return list(ts), strides[0]
    except ValueError:
        pass
    strides = []
    out = []
    for t, n in zip(ts, names):
        t, s = _rows_view(t, n)
        out.append(t)
        strides.append(s)
    if len(set(strides)) > 1:
        out = [t.contiguous() for t in out]
        strides = [_batch_stride(t, n) for t, n in zip(out, names)]
    return out, strides[0]


def _desc(B, T, D, DS, io, x_bs=0, bc_bs=0, y_bs=0) -> sscan_desc:
    d = sscan_desc()
    d.B, d.T, d.D, d.DS, d.io = int(B), int(T), int(D), int(DS), int(io)
    d.x_bstride, d.bc_bstride, d.y_bstride = int(x_bs), int(bc_bs), int(y_bs)
    return d


def _check_device(device: torch.device, **tensors):
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _f32_contig(t: Optional[torch.Tensor], shape, name):
    if t is None:
        return None
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.contiguous()


def _f32_out(t: Optional[torch.Tensor], shape, name):
    """A caller-supplied fp32 output: must already be float32, of ``shape`` and contiguous
    (the kernels write exactly that many fp32 values at its address)."""
    if t is None:
        return None
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)}, got "
                         f"{t.dtype} {tuple(t.shape)}{'' if t.is_contiguous() else ' (not contiguous)'}")
    return t


def sscan_version() -> int:
    return int(_lib.load().sscan_version())


def sscan_plan_select(B: int, T: int, D: int, DS: int, io: torch.dtype = torch.float32, backward: bool = False,
                      mamba: bool = False, with_H: bool = False, ckpt: bool = False) -> Plan:
    """The plan the library picks: the forward's (without H; ``with_H`` for the forward
    writing H, ``ckpt`` for the forward keeping boundary states), or with ``backward`` the
    backward's (with ``mamba`` that of the wrapper's backward)."""
    lib = _lib.load()
    d = _desc(B, T, D, DS, _IO[io])
    p = sscan_plan()
    if backward:
        kind = 2 if mamba else 1
    else:
        kind = 3 if with_H else (4 if ckpt else 0)
    _lib.check(lib.sscan_plan_select(ctypes.byref(d), kind, ctypes.byref(p)))
    return Plan(p.lanes, p.chunks, "state_groups" if p.layout == 2 else "lanes")


def sscan_fwd_workspace(B: int, T: int, D: int, DS: int, io: torch.dtype = torch.float32,
                        plan: Optional[Plan] = None) -> int:
    lib = _lib.load()
    d = _desc(B, T, D, DS, _IO[io])
    _, pp = _plan_ptr(plan)
    n = ctypes.c_size_t(0)
    _lib.check(lib.sscan_fwd_workspace(ctypes.byref(d), pp, ctypes.byref(n)))
    return int(n.value)


def sscan_bwd_workspace(B: int, T: int, D: int, DS: int, io: torch.dtype = torch.float32,
                        plan: Optional[Plan] = None) -> int:
    lib = _lib.load()
    d = _desc(B, T, D, DS, _IO[io])
    _, pp = _plan_ptr(plan)
    n = ctypes.c_size_t(0)
    _lib.check(lib.sscan_bwd_workspace(ctypes.byref(d), pp, ctypes.byref(n)))
    return int(n.value)


def sscan_mamba_bwd_workspace(B: int, T: int, D: int, DS: int, io: torch.dtype = torch.float32,
                              plan: Optional[Plan] = None) -> int:
    lib = _lib.load()
    d = _desc(B, T, D, DS, _IO[io])
    _, pp = _plan_ptr(plan)
    n = ctypes.c_size_t(0)
    _lib.check(lib.sscan_mamba_bwd_workspace(ctypes.byref(d), pp, ctypes.byref(n)))
    return int(n.value)


def _workspace(nbytes: int, device, given: Optional[torch.Tensor]):
    if nbytes == 0:
        return None, 0
    if given is not None:
        if given.device != device or given.numel() * given.element_size() < nbytes:
            raise ValueError(f"workspace must be a {nbytes}-byte buffer on {device}")
        return given, given.numel() * given.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def sscan_fwd(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, b: torch.Tensor, c: torch.Tensor,
              h0: Optional[torch.Tensor] = None, *, y: Optional[torch.Tensor] = None,
              hT: Optional[torch.Tensor] = None, H: Optional[torch.Tensor] = None, return_H: bool = False,
              plan: Optional[Plan] = None, workspace: Optional[torch.Tensor] = None):
    """Forward scan.  Returns (y, hT) or, with ``return_H`` (or ``H`` given), (y, hT, H).

    x, delta: (B,T,D) fp32 or bf16 (same dtype, may be T-slices of longer tensors);
    A: (D,DS) fp32; b, c: (B,T,DS) same dtype as x; h0: (B,D,DS) fp32 or None (zeros).
    y (optional out): (B,T,D) of x's dtype; hT (optional out): (B,D,DS) fp32;
    H (optional out): (B,T,D,DS) fp32 per-step states.
    """
    return _fwd_call(False, x, delta, A, b, c, None, h0, y, hT, H, return_H, plan, workspace)


def sscan_fwd_noalloc(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, b: torch.Tensor, c: torch.Tensor,
                      h0: Optional[torch.Tensor] = None, *, y: Optional[torch.Tensor] = None,
                      hT: Optional[torch.Tensor] = None, H: Optional[torch.Tensor] = None, return_H: bool = False,
                      plan: Optional[Plan] = None):
    """``sscan_fwd`` through the library's allocation-free entry point: its scratch is a
    static device array of the library (32 MiB per GPU), so the call itself allocates no
    device memory when ``y`` and ``hT`` (and ``H``) are supplied.  Calls that overlap in
    time on one GPU race on that array.  Same arguments and returns as ``sscan_fwd``."""
    return _fwd_call(False, x, delta, A, b, c, None, h0, y, hT, H, return_H, plan, None, noalloc=True)


def sscan_mamba_fwd(x: torch.Tensor, delta_raw: torch.Tensor, A_log: torch.Tensor, b: torch.Tensor,
                    c: torch.Tensor, Dskip: Optional[torch.Tensor] = None, h0: Optional[torch.Tensor] = None, *,
                    y: Optional[torch.Tensor] = None, hT: Optional[torch.Tensor] = None,
                    H: Optional[torch.Tensor] = None, return_H: bool = False, plan: Optional[Plan] = None,
                    workspace: Optional[torch.Tensor] = None):
    """Mamba-style wrapper: delta = softplus(delta_raw) (identity above 20), A = -exp(A_log),
    y = scan + Dskip * x.  Same shapes and returns as ``sscan_fwd``; Dskip: (D,) fp32 or None."""
    return _fwd_call(True, x, delta_raw, A_log, b, c, Dskip, h0, y, hT, H, return_H, plan, workspace)


def sscan_fwd_ckpt(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, b: torch.Tensor, c: torch.Tensor,
                   h0: Optional[torch.Tensor] = None, *, mamba: bool = False, Dskip: Optional[torch.Tensor] = None,
                   y: Optional[torch.Tensor] = None, hT: Optional[torch.Tensor] = None,
                   hck: Optional[torch.Tensor] = None, plan: Optional[Plan] = None,
                   workspace: Optional[torch.Tensor] = None):
    """Forward keeping boundary states instead of H.  Returns (y, hT, hck).

    hck: (B, ceil(T/32), D, DS) fp32, the state entering every 32-step block (hck[:, 0] = h0).
    With ``mamba`` the inputs are the wrapper's (delta_raw, A_log, Dskip) as in sscan_mamba_fwd.
    """
    return _fwd_call(mamba, x, delta, A, b, c, Dskip, h0, y, hT, None, False, plan, workspace, ckpt=True, hck=hck)


def _fwd_call(mamba, x, delta, A, b, c, Dskip, h0, y, hT, H, return_H, plan, workspace, ckpt=False, hck=None,
              noalloc=False):
    lib = _lib.load()
    if x.dtype not in _IO:
        raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")
    for n_, t in (("delta", delta), ("b", b), ("c", c)):
        if t.dtype != x.dtype:
            raise TypeError(f"{n_} must have x's dtype {x.dtype}, got {t.dtype}")
    device = x.device
    if device.type != "cuda":
        raise ValueError("sscan_fwd runs on a GPU: move the tensors to a HIP device")
    B, T, D = x.shape
    if A.dim() != 2 or A.shape[0] != D:
        raise ValueError(f"A must have shape (D, DS) with D={D}, got {tuple(A.shape)}")
    DS = A.shape[1]
    if tuple(delta.shape) != (B, T, D) or tuple(b.shape) != (B, T, DS) or tuple(c.shape) != (B, T, DS):
        raise ValueError("shape mismatch among x (B,T,D), delta (B,T,D), b and c (B,T,DS)")
    _check_device(device, delta=delta, A=A, b=b, c=c, h0=h0, y=y, hT=hT, H=H, Dskip=Dskip)
    (x, delta), x_bs = _same_stride([x, delta], ["x", "delta"])
    (b, c), bc_bs = _same_stride([b, c], ["b", "c"])
    A = _f32_contig(A, (D, DS), "A")
    h0 = _f32_contig(h0, (B, D, DS), "h0")
    Dskip = _f32_contig(Dskip, (D,), "Dskip")
    if y is None:
        y = torch.empty((B, T, D), dtype=x.dtype, device=device)
    elif y.dtype != x.dtype or tuple(y.shape) != (B, T, D):
        raise ValueError("y must have x's dtype and shape")
    y_bs = _batch_stride(y, "y")
    if hT is None:
        hT = torch.empty((B, D, DS), dtype=torch.float32, device=device)
    else:
        _f32_out(hT, (B, D, DS), "hT")
    if H is None and return_H:
        H = torch.empty((B, T, D, DS), dtype=torch.float32, device=device)
    _f32_out(H, (B, T, D, DS), "H")
    if ckpt:
        nck = (T + _lib.SSCAN_CKPT_STEPS - 1) // _lib.SSCAN_CKPT_STEPS
        if hck is None:
            hck = torch.empty((B, nck, D, DS), dtype=torch.float32, device=device)
        else:
            _f32_out(hck, (B, nck, D, DS), "hck")
    d = _desc(B, T, D, DS, _IO[x.dtype], x_bs, bc_bs, y_bs)
    pc, pp = _plan_ptr(plan)
    if noalloc:
        st = _call(device, lib.sscan_fwd_noalloc, ctypes.byref(d), pp, _ptr(x), _ptr(delta), _ptr(A), _ptr(b),
                   _ptr(c), _ptr(h0), _ptr(y), _ptr(hT), _ptr(H), _stream(device))
        _lib.check(st)
        return (y, hT, H) if (return_H or H is not None) else (y, hT)
    ws, wsn = _workspace(_ws_bytes(device, "fwd", lib.sscan_fwd_workspace, d, plan, pp), device, workspace)
    if ckpt:
        st = _call(device, lib.sscan_fwd_ckpt, ctypes.byref(d), pp, int(bool(mamba)), _ptr(x), _ptr(delta), _ptr(A),
                   _ptr(b), _ptr(c), _ptr(Dskip), _ptr(h0), _ptr(y), _ptr(hT), _ptr(hck), _ptr(ws), wsn,
                   _stream(device))
    elif mamba:
        st = _call(device, lib.sscan_mamba_fwd, ctypes.byref(d), pp, _ptr(x), _ptr(delta), _ptr(A), _ptr(b),
                   _ptr(c), _ptr(Dskip), _ptr(h0), _ptr(y), _ptr(hT), _ptr(H), _ptr(ws), wsn, _stream(device))
    else:
        st = _call(device, lib.sscan_fwd, ctypes.byref(d), pp, _ptr(x), _ptr(delta), _ptr(A), _ptr(b), _ptr(c),
                   _ptr(h0), _ptr(y), _ptr(hT), _ptr(H), _ptr(ws), wsn, _stream(device))
    _lib.check(st)
    if ckpt:
        return y, hT, hck
    return (y, hT, H) if (return_H or H is not None) else (y, hT)


def sscan_bwd(dy: torch.Tensor, x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, b: torch.Tensor,
              c: torch.Tensor, h0: Optional[torch.Tensor], H: torch.Tensor, dhT: Optional[torch.Tensor] = None, *,
              need_gh0: bool = True, plan: Optional[Plan] = None, workspace: Optional[torch.Tensor] = None,
              out: Optional[Tuple[torch.Tensor, ...]] = None):
    """Backward scan.  Returns (gx, gdelta, gb, gc, gA, gh0), all float32 (gh0 None if not needed).

    Gradients of sum(dy*y) + sum(dhT*hT); gb, gc are summed over channels and gA over
    batch rows and steps.  H is the (B,T,D,DS) state tensor the forward materialised.
    ``out`` may supply the six contiguous float32 output tensors (gh0 may be None).
    """
    return _bwd_call(False, dy, x, delta, A, b, c, None, h0, H, dhT, need_gh0, False, plan, workspace, out)


def sscan_mamba_bwd(dy: torch.Tensor, x: torch.Tensor, delta_raw: torch.Tensor, A_log: torch.Tensor,
                    b: torch.Tensor, c: torch.Tensor, Dskip: Optional[torch.Tensor], h0: Optional[torch.Tensor],
                    H: torch.Tensor, dhT: Optional[torch.Tensor] = None, *, need_gh0: bool = True,
                    need_gDskip: bool = True, plan: Optional[Plan] = None,
                    workspace: Optional[torch.Tensor] = None, out: Optional[Tuple[torch.Tensor, ...]] = None):
    """Backward of ``sscan_mamba_fwd``.  Returns (gx, gdelta_raw, gb, gc, gA_log, gh0, gDskip).

    gDskip (D,) is the gradient for Dskip (sum over b, t of dy*x), also when Dskip is None;
    None if not needed.  ``out`` may supply the seven outputs in that order.
    """
    return _bwd_call(True, dy, x, delta_raw, A_log, b, c, Dskip, h0, H, dhT, need_gh0, need_gDskip, plan,
                     workspace, out)


def sscan_bwd_ckpt(dy: torch.Tensor, x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, b: torch.Tensor,
                   c: torch.Tensor, hck: torch.Tensor, dhT: Optional[torch.Tensor] = None, *, mamba: bool = False,
                   Dskip: Optional[torch.Tensor] = None, need_gh0: bool = True, need_gDskip: bool = True,
                   plan: Optional[Plan] = None, workspace: Optional[torch.Tensor] = None,
                   out: Optional[Tuple[torch.Tensor, ...]] = None):
    """Backward from the boundary states of ``sscan_fwd_ckpt`` (no H).

    Returns what ``sscan_bwd`` returns, or with ``mamba`` what ``sscan_mamba_bwd`` returns.
    """
    return _bwd_call(mamba, dy, x, delta, A, b, c, Dskip, None, None, dhT, need_gh0, need_gDskip and mamba, plan,
                     workspace, out, hck=hck)


def _bwd_call(mamba, dy, x, delta, A, b, c, Dskip, h0, H, dhT, need_gh0, need_gD, plan, workspace, out, hck=None):
    lib = _lib.load()
    if x.dtype not in _IO:
        raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")
    for n_, t in (("dy", dy), ("delta", delta), ("b", b), ("c", c)):
        if t.dtype != x.dtype:
            raise TypeError(f"{n_} must have x's dtype {x.dtype}, got {t.dtype}")
    device = x.device
    if device.type != "cuda":
        raise ValueError("sscan_bwd runs on a GPU: move the tensors to a HIP device")
    B, T, D = x.shape
    DS = A.shape[1]
    if tuple(dy.shape) != (B, T, D) or tuple(delta.shape) != (B, T, D):
        raise ValueError("dy and delta must have x's shape")
    if tuple(b.shape) != (B, T, DS) or tuple(c.shape) != (B, T, DS):
        raise ValueError("b and c must have shape (B,T,DS)")
    _check_device(device, dy=dy, delta=delta, A=A, b=b, c=c, h0=h0, H=H, dhT=dhT, Dskip=Dskip)
    Dskip = _f32_contig(Dskip, (D,), "Dskip")
    (x, delta, dy), x_bs = _same_stride([x, delta, dy], ["x", "delta", "dy"])
    (b, c), bc_bs = _same_stride([b, c], ["b", "c"])
    A = _f32_contig(A, (D, DS), "A")
    h0 = _f32_contig(h0, (B, D, DS), "h0")
    dhT = _f32_contig(dhT, (B, D, DS), "dhT")
    ckpt = hck is not None
    if ckpt:
        nck = (T + _lib.SSCAN_CKPT_STEPS - 1) // _lib.SSCAN_CKPT_STEPS
        hck = _f32_contig(hck, (B, nck, D, DS), "hck")
        if H is not None:
            raise ValueError("H and hck are alternatives")
    else:
        H = _f32_contig(H, (B, T, D, DS), "H")
    f32 = dict(dtype=torch.float32, device=device)
    gD = None
    if out is not None:
        if mamba:
            gx, gdelta, gb, gc, gA, gh0, gD = out
        else:
            gx, gdelta, gb, gc, gA, gh0 = out
        shapes = [(B, T, D), (B, T, D), (B, T, DS), (B, T, DS), (D, DS), (B, D, DS), (D,)]
        for name, t, shp in zip(["gx", "gdelta", "gb", "gc", "gA", "gh0", "gDskip"], out, shapes):
            if t is None and name in ("gh0", "gDskip"):
                continue
            if t is None or t.dtype != torch.float32 or tuple(t.shape) != shp or not t.is_contiguous() \
                    or t.device != device:
                raise ValueError(f"out {name} must be a contiguous float32 tensor of shape {shp} on {device}")
    else:
        gx = torch.empty((B, T, D), **f32)
        gdelta = torch.empty((B, T, D), **f32)
        gb = torch.empty((B, T, DS), **f32)
        gc = torch.empty((B, T, DS), **f32)
        gA = torch.empty((D, DS), **f32)
        gh0 = torch.empty((B, D, DS), **f32) if need_gh0 else None
        gD = torch.empty((D,), **f32) if (mamba and need_gD) else None
    d = _desc(B, T, D, DS, _IO[x.dtype], x_bs, bc_bs, 0)
    pc, pp = _plan_ptr(plan)
    if ckpt:
        nws = _ws_bytes(device, "bwd_ckpt", lib.sscan_bwd_ckpt_workspace, d, plan, pp, int(bool(mamba)))
    elif mamba:
        nws = _ws_bytes(device, "mamba_bwd", lib.sscan_mamba_bwd_workspace, d, plan, pp)
    else:
        nws = _ws_bytes(device, "bwd", lib.sscan_bwd_workspace, d, plan, pp)
    ws, wsn = _workspace(nws, device, workspace)
    if ckpt:
        st = _call(device, lib.sscan_bwd_ckpt, ctypes.byref(d), pp, int(bool(mamba)), _ptr(dy), _ptr(dhT), _ptr(x),
                   _ptr(delta), _ptr(A), _ptr(b), _ptr(c), _ptr(Dskip), _ptr(hck), _ptr(gx), _ptr(gdelta), _ptr(gb),
                   _ptr(gc), _ptr(gA), _ptr(gD), _ptr(gh0), _ptr(ws), wsn, _stream(device))
    elif mamba:
        st = _call(device, lib.sscan_mamba_bwd, ctypes.byref(d), pp, _ptr(dy), _ptr(dhT), _ptr(x), _ptr(delta),
                   _ptr(A), _ptr(b), _ptr(c), _ptr(Dskip), _ptr(h0), _ptr(H), _ptr(gx), _ptr(gdelta), _ptr(gA),
                   _ptr(gb), _ptr(gc), _ptr(gD), _ptr(gh0), _ptr(ws), wsn, _stream(device))
    else:
        st = _call(device, lib.sscan_bwd, ctypes.byref(d), pp, _ptr(dy), _ptr(dhT), _ptr(x), _ptr(delta), _ptr(A),
                   _ptr(b), _ptr(c), _ptr(h0), _ptr(H), _ptr(gx), _ptr(gdelta), _ptr(gb), _ptr(gc), _ptr(gA),
                   _ptr(gh0), _ptr(ws), wsn, _stream(device))
    _lib.check(st)
    if mamba:
        return gx, gdelta, gb, gc, gA, gh0, gD
    return gx, gdelta, gb, gc, gA, gh0


def sscan_decode(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, b: torch.Tensor, c: torch.Tensor,
                 state: torch.Tensor, *, y: Optional[torch.Tensor] = None, state_out: Optional[torch.Tensor] = None,
                 inplace: bool = False):
    """One decode step on a resident state.  Returns (y, state_out).

    x, delta: (B,D) or (B,1,D) fp32 or bf16; A: (D,DS) fp32; b, c: (B,DS) or (B,1,DS) of x's
    dtype; state: (B,D,DS) contiguous fp32.  With ``inplace`` the new state overwrites
    ``state`` (and is returned); otherwise it goes to ``state_out`` (allocated if None).
    y has x's dtype and shape.
    """
    lib = _lib.load()
    if x.dtype not in _IO:
        raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")
    for n_, t in (("delta", delta), ("b", b), ("c", c)):
        if t.dtype != x.dtype:
            raise TypeError(f"{n_} must have x's dtype {x.dtype}, got {t.dtype}")
    device = x.device
    if device.type != "cuda":
        raise ValueError("sscan_decode runs on a GPU: move the tensors to a HIP device")
    squeeze = x.dim() == 2
    x3, d3 = (x.unsqueeze(1), delta.unsqueeze(1)) if squeeze else (x, delta)
    b3 = b.unsqueeze(1) if b.dim() == 2 else b
    c3 = c.unsqueeze(1) if c.dim() == 2 else c
    if x3.dim() != 3 or x3.shape[1] != 1:
        raise ValueError(f"x must be (B,D) or (B,1,D), got {tuple(x.shape)}")
    B, _, D = x3.shape
    if A.dim() != 2 or A.shape[0] != D:
        raise ValueError(f"A must have shape (D, DS) with D={D}, got {tuple(A.shape)}")
    DS = A.shape[1]
    if tuple(d3.shape) != (B, 1, D) or tuple(b3.shape) != (B, 1, DS) or tuple(c3.shape) != (B, 1, DS):
        raise ValueError("shape mismatch among x, delta (B,D) and b, c (B,DS)")
    _check_device(device, delta=delta, A=A, b=b, c=c, state=state, y=y, state_out=state_out)
    (x3, d3), x_bs = _same_stride([x3, d3], ["x", "delta"])
    (b3, c3), bc_bs = _same_stride([b3, c3], ["b", "c"])
    A = _f32_contig(A, (D, DS), "A")
    if state.dtype != torch.float32 or tuple(state.shape) != (B, D, DS) or not state.is_contiguous():
        raise ValueError(f"state must be a contiguous float32 tensor of shape {(B, D, DS)}")
    if inplace:
        state_out = state
    elif state_out is None:
        state_out = torch.empty_like(state)
    elif state_out.dtype != torch.float32 or tuple(state_out.shape) != (B, D, DS) or not state_out.is_contiguous():
        raise ValueError(f"state_out must be a contiguous float32 tensor of shape {(B, D, DS)}")
    y3 = torch.empty((B, 1, D), dtype=x.dtype, device=device) if y is None else (y.unsqueeze(1) if y.dim() == 2 else y)
    if y3.dtype != x.dtype or tuple(y3.shape) != (B, 1, D):
        raise ValueError("y must have x's dtype and shape")
    y_bs = _batch_stride(y3, "y")
    d = _desc(B, 1, D, DS, _IO[x.dtype], x_bs, bc_bs, y_bs)
    st = _call(device, lib.sscan_decode, ctypes.byref(d), _ptr(x3), _ptr(d3), _ptr(A), _ptr(b3), _ptr(c3),
               _ptr(state), _ptr(state_out), _ptr(y3), _stream(device))
    _lib.check(st)
    return (y3.squeeze(1) if squeeze else y3), state_out


class SelectiveScan(torch.autograd.Function):
    """Differentiable scan: (x, delta, A, b, c, h0) -> (y, hT), with gradients for hT too.

    The forward keeps the per-step states H for a single reverse sweep in the backward.
    """

    @staticmethod
    def forward(ctx, x, delta, A, b, c, h0=None, ckpt=False):
        if ckpt:
            y, hT, S = sscan_fwd_ckpt(x, delta, A, b, c, h0)
        else:
            y, hT, S = sscan_fwd(x, delta, A, b, c, h0, return_H=True)
        ctx.save_for_backward(x, delta, A, b, c, h0, S)
        ctx.has_h0 = h0 is not None
        ctx.ckpt = ckpt
        return y, hT

    @staticmethod
    def backward(ctx, dy, dhT):
        x, delta, A, b, c, h0, S = ctx.saved_tensors
        if dy is None:
            dy = torch.zeros_like(x)
        dy = dy.to(x.dtype)
        dhT = None if dhT is None else dhT.float().contiguous()
        if ctx.ckpt:
            gx, gdelta, gb, gc, gA, gh0 = sscan_bwd_ckpt(dy, x, delta, A, b, c, S, dhT, need_gh0=ctx.has_h0)
        else:
            gx, gdelta, gb, gc, gA, gh0 = sscan_bwd(dy, x, delta, A, b, c, h0, S, dhT, need_gh0=ctx.has_h0)
        return (gx.to(x.dtype), gdelta.to(delta.dtype), gA, gb.to(b.dtype), gc.to(c.dtype),
                gh0 if ctx.has_h0 else None, None)


def selective_scan(x, delta, A, b, c, h0=None, ckpt=False):
    """Autograd-aware forward: returns (y, hT).  ``ckpt`` keeps boundary states instead of H
    (1/32 of the memory; the backward recomputes the states)."""
    return SelectiveScan.apply(x, delta, A, b, c, h0, ckpt)


class MambaScan(torch.autograd.Function):
    """Differentiable Mamba-style wrapper: (x, delta_raw, A_log, b, c, Dskip, h0) -> (y, hT)."""

    @staticmethod
    def forward(ctx, x, delta_raw, A_log, b, c, Dskip=None, h0=None, ckpt=False):
        if ckpt:
            y, hT, S = sscan_fwd_ckpt(x, delta_raw, A_log, b, c, h0, mamba=True, Dskip=Dskip)
        else:
            y, hT, S = sscan_mamba_fwd(x, delta_raw, A_log, b, c, Dskip, h0, return_H=True)
        ctx.save_for_backward(x, delta_raw, A_log, b, c, Dskip, h0, S)
        ctx.has_h0 = h0 is not None
        ctx.has_D = Dskip is not None
        ctx.ckpt = ckpt
        return y, hT

    @staticmethod
    def backward(ctx, dy, dhT):
        x, delta_raw, A_log, b, c, Dskip, h0, S = ctx.saved_tensors
        if dy is None:
            dy = torch.zeros_like(x)
        dy = dy.to(x.dtype)
        dhT = None if dhT is None else dhT.float().contiguous()
        if ctx.ckpt:
            gx, gdr, gb, gc, gAl, gh0, gD = sscan_bwd_ckpt(dy, x, delta_raw, A_log, b, c, S, dhT, mamba=True,
                                                           Dskip=Dskip, need_gh0=ctx.has_h0,
                                                           need_gDskip=ctx.has_D)
        else:
            gx, gdr, gb, gc, gAl, gh0, gD = sscan_mamba_bwd(dy, x, delta_raw, A_log, b, c, Dskip, h0, S, dhT,
                                                            need_gh0=ctx.has_h0, need_gDskip=ctx.has_D)
        return (gx.to(x.dtype), gdr.to(delta_raw.dtype), gAl, gb.to(b.dtype), gc.to(c.dtype),
                gD if ctx.has_D else None, gh0 if ctx.has_h0 else None, None)


def mamba_scan(x, delta_raw, A_log, b, c, Dskip=None, h0=None, ckpt=False):
    """Autograd-aware Mamba-style wrapper: returns (y, hT); ``ckpt`` as in selective_scan."""
    return MambaScan.apply(x, delta_raw, A_log, b, c, Dskip, h0, ckpt)
