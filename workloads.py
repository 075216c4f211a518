"""Seeded synthetic inputs for the selective diagonal state-space scan.

This module is the only thing the GPU path and the fp64 oracle share.  It
draws inputs; it holds none of the scan's arithmetic.  Every array is built
on the CPU with ``torch.Generator().manual_seed(seed)`` in a fixed draw order
(x, delta_raw, b, c, A_u, h0, dy, dhT), all fp32, then:

* ``delta = softplus(delta_raw)`` with ``delta_raw ~ N(mu, 1)`` (positive steps);
* ``A[d, n] = -(n + 1) * U(0.5, 1.5)`` ("scaled") or ``-(n + 1)`` ("ladder"),
  or ``-softplus(N(0, 1))`` ("softplus", the shape of the pssa_kernels.py
  page's selftest);
* ``h0 = h0_std * N(0, 1)`` (absent, i.e. zeros, when ``h0_std == 0``);
* for bf16 workloads x, delta, b, c (and dy) are rounded to bf16 (round to
  nearest even) and those rounded values are what both sides consume.

The named workloads are the five sizes the scan is measured on plus the
selftest shape of the pssa_kernels.py page (B=2, T=7, D=64, DS=16).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    D: int
    DS: int
    io: str = "f32"            # "f32" or "bf16": dtype of x, delta, b, c, y, dy
    delta_mu: float = -2.0     # delta = softplus(N(delta_mu, 1))
    A_kind: str = "scaled"     # "scaled" | "ladder" | "softplus"
    h0_std: float = 0.0        # 0 => h0 is absent (zeros)
    with_dy: bool = False
    with_dhT: bool = False
    chunks: int = 1            # number of calls the sequence is split into (state carried)
    seed: int = 0
    note: str = ""

    @property
    def elems(self) -> int:
        return self.B * self.T * self.D


WORKLOADS: Dict[str, Workload] = {
    "tiny_fwd": Workload("tiny_fwd", 1, 64, 16, 4, "f32", delta_mu=-1.0, A_kind="ladder", seed=1,
                         note="B=1 T=64 D=16 DS=4 fp32, A[d,n]=-(n+1), h0=0"),
    "fwd_f32": Workload("fwd_f32", 8, 1024, 256, 16, "f32", seed=2,
                        note="B=8 T=1024 D=256 DS=16 fp32, h0=0"),
    "fwd_bf16": Workload("fwd_bf16", 16, 4096, 1024, 16, "bf16", h0_std=0.1, seed=3,
                         note="B=16 T=4096 D=1024 DS=16 bf16 I/O, fp32 state, h0~N(0,0.1)"),
    "long_chunked_bf16": Workload("long_chunked_bf16", 4, 16384, 2048, 16, "bf16", h0_std=0.1, chunks=8, seed=4,
                                  note="B=4 T=16384 D=2048 DS=16 bf16 I/O as 8 calls of T=2048, hT->h0"),
    "fwd_bwd_f32": Workload("fwd_bwd_f32", 8, 2048, 768, 16, "f32", h0_std=0.1, with_dy=True, seed=5,
                            note="B=8 T=2048 D=768 DS=16 fp32, H materialised, 6 gradients"),
    "selftest": Workload("selftest", 2, 7, 64, 16, "f32", delta_mu=0.0, A_kind="softplus", h0_std=0.5,
                         with_dy=True, seed=1,
                         note="B=2 T=7 D=64 DS=16 fp32, the pssa_kernels.py selftest shape"),
}


def get(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


def custom(B: int, T: int, D: int, DS: int, *, io: str = "f32", seed: int = 0, **kw) -> Workload:
    return Workload(f"custom_{B}x{T}x{D}x{DS}_{io}_{seed}", B, T, D, DS, io, seed=seed, **kw)


def _round_bf16(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.bfloat16)


def make_inputs(w: Workload) -> Dict[str, Optional[torch.Tensor]]:
    """Draw the inputs of workload ``w`` on the CPU.

    Returns a dict with keys x, delta, A, b, c, h0, dy, dhT, and for the
    Mamba-style wrapper delta_raw (delta = softplus(delta_raw)), A_log
    (A = -exp(A_log)) and Dskip (D,) ~ 1 + 0.5 N(0, 1).  x, delta, delta_raw, b,
    c (and dy) are fp32 for f32 workloads and bf16 for bf16 workloads; A, A_log,
    Dskip, h0 and dhT are always fp32.  h0 / dy / dhT are None when the workload
    has none.
    """
    g = torch.Generator().manual_seed(int(w.seed))
    B, T, D, DS = w.B, w.T, w.D, w.DS
    x = torch.randn(B, T, D, generator=g)
    delta_raw = torch.randn(B, T, D, generator=g) + w.delta_mu
    b = torch.randn(B, T, DS, generator=g)
    c = torch.randn(B, T, DS, generator=g)
    if w.A_kind == "softplus":
        A_u = torch.randn(D, DS, generator=g)
    else:
        A_u = torch.rand(D, DS, generator=g)
    h0_raw = torch.randn(B, D, DS, generator=g)
    dy = torch.randn(B, T, D, generator=g) if w.with_dy else None
    dhT = torch.randn(B, D, DS, generator=g) if w.with_dhT else None
    Dskip = 1.0 + 0.5 * torch.randn(D, generator=g)  # drawn last: the draws above are unchanged

    delta = torch.nn.functional.softplus(delta_raw)
    ladder = -torch.arange(1, DS + 1, dtype=torch.float32).expand(D, DS)
    if w.A_kind == "scaled":
        A = ladder * (0.5 + A_u)
    elif w.A_kind == "ladder":
        A = ladder.clone()
    elif w.A_kind == "softplus":
        A = -torch.nn.functional.softplus(A_u)
    else:
        raise ValueError(f"unknown A_kind {w.A_kind!r}")
    A = A.contiguous()
    h0 = (h0_raw * w.h0_std).contiguous() if w.h0_std > 0 else None

    A_log = torch.log(-A).contiguous()  # the Mamba-style parameterisation A = -exp(A_log)

    if w.io == "bf16":
        x, delta, delta_raw, b, c = (_round_bf16(t) for t in (x, delta, delta_raw, b, c))
        if dy is not None:
            dy = _round_bf16(dy)
    elif w.io != "f32":
        raise ValueError(f"unknown io dtype {w.io!r}")
    return {"x": x.contiguous(), "delta": delta.contiguous(), "A": A, "b": b.contiguous(),
            "c": c.contiguous(), "h0": h0, "dy": None if dy is None else dy.contiguous(), "dhT": dhT,
            "delta_raw": delta_raw.contiguous(), "A_log": A_log, "Dskip": Dskip.contiguous()}


def chunk_bounds(T: int, chunks: int):
    """Split [0, T) into ``chunks`` nearly equal consecutive ranges."""
    chunks = max(1, int(chunks))
    edges = [round(i * T / chunks) for i in range(chunks + 1)]
    return [(edges[i], edges[i + 1]) for i in range(chunks)]
