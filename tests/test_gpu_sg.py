"""GPU parity of the state-group forward layout (Plan(layout="state_groups"): one channel
per lane, a channel's states across the waves of its workgroup, 64 or 32 channels per
workgroup by the workgroup count) against the fp64 oracle on
the same seeded inputs, and against the lanes layout: its states come from the same
operations in the same order, so hT, H and the boundary states of the H-free path agree bit
for bit on a single pass; y differs only in the order of the sum over states.
Tolerances: 1e-4 (fp32 I/O), 2e-2 (bf16 I/O), norm-wise per tensor."""
import pytest
import torch

import oracle
import workloads
from parity import TOL_F32, announce, assert_close, rel_err, to_dev, tol_for

pytestmark = pytest.mark.gpu

sscan = pytest.importorskip("selective_state_space_sscan_amd")
from selective_state_space_sscan_amd import Plan, sscan_fwd, sscan_fwd_ckpt, sscan_mamba_fwd  # noqa: E402

SG = "state_groups"

CASES = [
    # B, T, D, DS, io, h0, chunks
    (2, 100, 64, 16, "f32", True, 1),
    (3, 77, 100, 16, "bf16", True, 1),    # ragged T and D (a partial 64-channel tile)
    (1, 300, 8, 8, "f32", False, 1),
    (2, 129, 12, 4, "f32", True, 1),
    (2, 1000, 68, 16, "f32", True, 4),    # two-level scan: chunks of whole 64-step tiles
    (1, 513, 40, 16, "bf16", True, 3),
    (1, 1, 4, 4, "f32", True, 1),
    (2, 64, 128, 16, "f32", True, 1),     # exactly one tile
    (2, 1024, 512, 16, "f32", True, 16),  # 256 workgroups: 64 channels per workgroup (32 otherwise)
]


def inputs(B, T, D, DS, io, h0, seed):
    w = workloads.custom(B, T, D, DS, io=io, seed=seed, h0_std=0.3 if h0 else 0.0, delta_mu=-1.0)
    return workloads.make_inputs(w)


@pytest.mark.parametrize("B,T,D,DS,io,h0,chunks", CASES)
def test_state_groups_forward_matches_oracle_and_lanes_layout(gpu, B, T, D, DS, io, h0, chunks):
    announce(f"state-group fwd B={B} T={T} D={D} DS={DS} io={io} h0={h0} chunks={chunks}")
    inp = inputs(B, T, D, DS, io, h0, seed=41 + T + D)
    g = to_dev(inp, gpu)
    y, hT = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], plan=Plan(0, chunks, SG))
    torch.cuda.synchronize()
    yr, hTr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"])
    assert_close("y", y, yr, tol_for(io))
    assert_close("hT", hT, hTr, TOL_F32)
    y1, hT1 = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], plan=Plan(0, chunks, "lanes"))
    torch.cuda.synchronize()
    assert rel_err(y.float(), y1.float()) < (1e-6 if io == "f32" else 1e-2)
    if chunks == 1:
        assert torch.equal(hT, hT1)  # the same fma chain per state
    else:
        assert rel_err(hT, hT1) < 1e-6


@pytest.mark.parametrize("B,T,D,DS,io,chunks", [(2, 300, 64, 16, "f32", 1), (2, 700, 36, 8, "bf16", 3)])
def test_state_groups_boundary_states(gpu, B, T, D, DS, io, chunks):
    announce(f"state-group fwd with boundary states B={B} T={T} D={D} DS={DS} io={io} chunks={chunks}")
    inp = inputs(B, T, D, DS, io, True, seed=5 + T)
    g = to_dev(inp, gpu)
    y, hT, hck = sscan_fwd_ckpt(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], plan=Plan(0, chunks, SG))
    y1, hT1, H = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], return_H=True)
    torch.cuda.synchronize()
    yr, hTr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"])
    assert_close("y", y, yr, tol_for(io))
    CK = 32
    assert torch.equal(hck[:, 0], g["h0"])
    # the state entering block k is H after step 32k - 1
    ref_ck = H[:, CK - 1::CK][:, : hck.shape[1] - 1]
    if chunks == 1:
        assert torch.equal(hck[:, 1:], ref_ck) and torch.equal(hT, hT1)
    else:  # the chunk carries compose decay products, rounded differently from the single pass
        assert rel_err(hck[:, 1:], ref_ck) < 1e-6 and rel_err(hT, hT1) < 1e-6


@pytest.mark.parametrize("B,T,D,DS,io,with_D", [(2, 150, 64, 16, "f32", True), (1, 90, 20, 4, "bf16", False)])
def test_state_groups_mamba_wrapper(gpu, B, T, D, DS, io, with_D):
    announce(f"state-group mamba fwd B={B} T={T} D={D} DS={DS} io={io} Dskip={with_D}")
    w = workloads.custom(B, T, D, DS, io=io, seed=77 + T, h0_std=0.3, delta_mu=-1.0)
    inp = workloads.make_inputs(w)
    raw = inp["delta_raw"].clone()
    raw[0, 1, : min(3, D)] = 21.0  # the identity branch of the softplus
    inp["delta_raw"] = raw
    g = to_dev(inp, gpu)
    Dk = g["Dskip"] if with_D else None
    y, hT = sscan_mamba_fwd(g["x"], g["delta_raw"], g["A_log"], g["b"], g["c"], Dk, g["h0"], plan=Plan(0, 1, SG))
    torch.cuda.synchronize()
    yr, hTr = oracle.mamba_fwd(inp["x"], inp["delta_raw"], inp["A_log"], inp["b"], inp["c"],
                               inp["Dskip"] if with_D else None, inp["h0"])
    assert_close("y", y, yr, tol_for(io))
    assert_close("hT", hT, hTr, TOL_F32)


H_CASES = [
    # B, T, D, io, h0, chunks (DS = 16: 32-channel workgroups, 16-step tiles)
    (2, 100, 64, "f32", True, 1),       # ragged T: the last tile partly past the end
    (3, 77, 100, "bf16", True, 1),      # ragged D: a partial 32-channel tile
    (2, 1000, 68, "f32", True, 4),      # two-level scan: chunks of whole 64-step tiles
    (1, 16, 32, "f32", False, 1),       # exactly one tile
    (1, 1, 4, "f32", True, 1),
    (4, 300, 1024, "bf16", False, 1),   # 128 workgroups, the size class the library picks it for
]


@pytest.mark.parametrize("B,T,D,io,h0,chunks", H_CASES)
def test_state_groups_write_H(gpu, B, T, D, io, h0, chunks):
    DS = 16
    announce(f"state-group fwd writing H B={B} T={T} D={D} DS={DS} io={io} h0={h0} chunks={chunks}")
    inp = inputs(B, T, D, DS, io, h0, seed=91 + T + D)
    g = to_dev(inp, gpu)
    y, hT, H = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], return_H=True,
                         plan=Plan(0, chunks, SG))
    torch.cuda.synchronize()
    yr, hTr, Hr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], return_H=True)
    assert_close("y", y, yr, tol_for(io))
    assert_close("hT", hT, hTr, TOL_F32)
    assert_close("H", H, Hr, TOL_F32)
    y1, hT1, H1 = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], return_H=True,
                            plan=Plan(0, chunks, "lanes"))
    torch.cuda.synchronize()
    assert rel_err(y.float(), y1.float()) < (1e-6 if io == "f32" else 1e-2)
    if chunks == 1:
        assert torch.equal(H, H1) and torch.equal(hT, hT1)  # the same fma chain per state
    else:  # the layouts split the sequence at different steps
        assert rel_err(H, H1) < 1e-6 and rel_err(hT, hT1) < 1e-6


def test_state_groups_write_H_mamba_wrapper(gpu):
    B, T, D, DS = 2, 150, 96, 16
    announce(f"state-group mamba fwd writing H B={B} T={T} D={D} DS={DS}")
    w = workloads.custom(B, T, D, DS, io="f32", seed=17, h0_std=0.3, delta_mu=-1.0)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    args = (g["x"], g["delta_raw"], g["A_log"], g["b"], g["c"], g["Dskip"], g["h0"])
    y, hT, H = sscan_mamba_fwd(*args, return_H=True, plan=Plan(0, 1, SG))
    y1, hT1, H1 = sscan_mamba_fwd(*args, return_H=True, plan=Plan(0, 1, "lanes"))
    torch.cuda.synchronize()
    yr, hTr = oracle.mamba_fwd(inp["x"], inp["delta_raw"], inp["A_log"], inp["b"], inp["c"], inp["Dskip"], inp["h0"])
    assert_close("y", y, yr, TOL_F32)
    assert_close("hT", hT, hTr, TOL_F32)
    assert torch.equal(H, H1) and torch.equal(hT, hT1)
    assert rel_err(y, y1) < 1e-6


def test_default_plan_picks_state_groups_for_many_channels(gpu):
    announce("default plan: 16x512x1024x16 bf16 runs the state-group layout")
    inp = inputs(16, 512, 1024, 16, "bf16", True, seed=3)
    g = to_dev(inp, gpu)
    y, hT = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"])
    y1, hT1 = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], plan=Plan(0, 1, SG))
    torch.cuda.synchronize()
    assert torch.equal(y, y1) and torch.equal(hT, hT1)


def test_default_plan_writes_H_in_state_groups(gpu):
    announce("default plan: 8x256x768x16 fp32 writing H runs the state-group layout")
    inp = inputs(8, 256, 768, 16, "f32", True, seed=4)
    g = to_dev(inp, gpu)
    out = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], return_H=True)
    out1 = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], return_H=True, plan=Plan(0, 1, SG))
    torch.cuda.synchronize()
    for a, b in zip(out, out1):
        assert torch.equal(a, b)


def test_state_groups_write_H_full_size_bitwise(gpu):
    """At the fwd+bwd workload's full size (8x2048x768x16 fp32, 805 MB of H) the state-group
    forward writing H, the library's choice there, gives every state and hT bit for bit as
    the lanes layout, and y within fp32 rounding of it (the sum over states runs in another
    order); both are checked against the fp64 oracle by the full-size parity test."""
    w = workloads.get("fwd_bwd_f32")
    announce(f"{w.name}: state groups vs lanes, H bitwise at full size")
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    args = (g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"])
    y, hT, H = sscan_fwd(*args, return_H=True, plan=Plan(0, 1, SG))
    torch.cuda.synchronize()
    H_sg = H.cpu()
    del H
    y1, hT1, H1 = sscan_fwd(*args, return_H=True, plan=Plan(0, 1, "lanes"))
    torch.cuda.synchronize()
    assert torch.equal(hT, hT1)
    assert torch.equal(H_sg, H1.cpu())
    assert rel_err(y, y1) < 1e-6


def test_state_groups_write_H_added_tiles_read_zeros(gpu):
    """MODE 3 rounds its 16-step tiles up to whole 128-step staging tiles: at T = 130 the packed
    b/c rows hold 192 steps and the added tiles run to step 256.  Those tiles must read zeros
    for b and c, not the next state group's packed values: with b infinite in state 2 (state
    group 1) at step 5, states 0 and 1 (group 0) stay finite and bitwise the lanes layout's."""
    B, T, D, DS = 1, 130, 32, 16
    announce(f"state-group fwd writing H, B={B} T={T} D={D}: added tiles past the packed rows")
    inp = inputs(B, T, D, DS, "f32", True, seed=23)
    b = inp["b"].clone()
    b[0, 5, 2] = float("inf")
    inp["b"] = b
    g = to_dev(inp, gpu)
    args = (g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"])
    _, hT, H = sscan_fwd(*args, return_H=True, plan=Plan(0, 1, SG))
    _, hT1, H1 = sscan_fwd(*args, return_H=True, plan=Plan(0, 1, "lanes"))
    torch.cuda.synchronize()
    assert torch.isfinite(hT[..., :2]).all() and torch.isfinite(H[..., :2]).all()
    assert torch.equal(hT[..., :2], hT1[..., :2]) and torch.equal(H[..., :2], H1[..., :2])
    assert not torch.isfinite(hT[..., 2]).all()  # the state the infinite b feeds
