"""The allocation-free forward (sscan_fwd_noalloc) against the forward that takes a
caller workspace (sscan_fwd): the same kernels on the same inputs, so the outputs must
be bitwise equal, and both within the fp32 / bf16 tolerance of the fp64 oracle.  Two
calls in a row, the second on a smaller problem, so the second reads a scratch array
that still holds the first call's data."""
import pytest
import torch

import oracle
import workloads
from parity import TOL_F32, announce, assert_close, to_dev, tol_for

pytestmark = pytest.mark.gpu

sscan = pytest.importorskip("selective_state_space_sscan_amd")
from selective_state_space_sscan_amd import (Plan, SScanError, sscan_fwd, sscan_fwd_noalloc,  # noqa: E402
                                             sscan_fwd_workspace, sscan_plan_select)
from selective_state_space_sscan_amd import _lib  # noqa: E402

CALLS = [
    # B, T, D, DS, io, plan (lanes, chunks, layout), with_H
    (8, 600, 1024, 16, "f32", (0, 0, None), True),              # writing H through the state-group layout
    (1, 4096, 256, 16, "f32", (0, 0, None), False),             # the library's plan: state groups in 16 T-chunks
    (4, 1000, 256, 16, "bf16", (0, 0, "state_groups"), False),  # packed b/c in the scratch (~2 MB)
    (2, 300, 70, 16, "f32", (8, 3, "lanes"), False),            # carry pairs of a 3-chunk two-level scan
    (1, 129, 33, 8, "f32", (0, 0, None), True),                 # the library's own plan, writing H
]


def _one(gpu, B, T, D, DS, io, plan, with_H, seed):
    w = workloads.custom(B, T, D, DS, io=io, seed=seed, h0_std=0.3, delta_mu=-1.0)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    pl = Plan(*plan)
    need = sscan_fwd_workspace(B, T, D, DS, g["x"].dtype, pl)
    assert 0 < need <= _lib.SSCAN_NOALLOC_SCRATCH_BYTES or (need == 0 and plan[2] is None)
    if DS == 16 and plan[2] is None and D >= 256:  # the library's plan takes state groups here
        assert sscan_plan_select(B, T, D, DS, g["x"].dtype, with_H=with_H).layout == "state_groups"
    ref = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], plan=pl, return_H=with_H)
    y = torch.full_like(g["x"], float("nan"))
    hT = torch.full((B, D, DS), float("nan"), device=gpu)
    H = torch.full((B, T, D, DS), float("nan"), device=gpu) if with_H else None
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated(gpu)
    got = sscan_fwd_noalloc(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], y=y, hT=hT, H=H, plan=pl)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated(gpu) == before  # outputs supplied: nothing allocated through torch
    for name, a, r in zip(["y", "hT", "H"], got, ref):
        assert torch.equal(a, r), name
    yr, hTr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"])
    assert_close("y", got[0], yr, tol_for(io))
    assert_close("hT", got[1], hTr, TOL_F32)


def test_noalloc_forward_two_calls_in_a_row(gpu):
    for k, (B, T, D, DS, io, plan, with_H) in enumerate(CALLS):
        announce(f"noalloc fwd call {k}: B={B} T={T} D={D} DS={DS} io={io} plan={plan} H={with_H}")
        _one(gpu, B, T, D, DS, io, plan, with_H, seed=60 + k)


def test_noalloc_forward_rejects_more_than_its_scratch(gpu):
    # the state-group layout packs B*T*2*DS floats of b and c: 64 x 65536 x 32 x 4 B = 512 MiB
    B, T, D, DS = 64, 65536, 4, 16
    announce("noalloc fwd beyond its scratch: expect SSCAN_ERR_WORKSPACE before any launch")
    x = torch.zeros(B, T, D, device=gpu)
    bc = torch.zeros(B, T, DS, device=gpu)
    A = -torch.ones(D, DS, device=gpu)
    with pytest.raises(SScanError, match="SSCAN_ERR_WORKSPACE"):
        sscan_fwd_noalloc(x, x, A, bc, bc, plan=Plan(0, 1, "state_groups"))


def test_noalloc_forward_writing_H_beyond_its_scratch_runs_the_lanes_layout(gpu):
    # 128 x 2100 x 64 x 16 writing H: the library's plan, one state-group pass (256
    # workgroups of 32 channels), would pack 128 * 2100 * 128 B = 34.4 MB of b and c, more
    # than the 32 MiB array; the allocation-free call runs the lanes layout instead, whose
    # states and outputs are those of sscan_fwd with a lanes plan, bit for bit
    B, T, D, DS = 128, 2100, 64, 16
    announce(f"noalloc fwd writing H, B={B} T={T} D={D} DS={DS}: lanes layout within the scratch")
    w = workloads.custom(B, T, D, DS, io="f32", seed=71, h0_std=0.3, delta_mu=-1.0)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    assert sscan_fwd_workspace(B, T, D, DS, g["x"].dtype, None) > _lib.SSCAN_NOALLOC_SCRATCH_BYTES
    ref = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], plan=Plan(0, 0, "lanes"), return_H=True)
    y = torch.full_like(g["x"], float("nan"))
    hT = torch.full((B, D, DS), float("nan"), device=gpu)
    H = torch.full((B, T, D, DS), float("nan"), device=gpu)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated(gpu)
    got = sscan_fwd_noalloc(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], y=y, hT=hT, H=H)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated(gpu) == before
    for name, a, r in zip(["y", "hT", "H"], got, ref):
        assert torch.equal(a, r), name
    yr, hTr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"])
    assert_close("y", got[0], yr, TOL_F32)
    assert_close("hT", got[1], hTr, TOL_F32)
