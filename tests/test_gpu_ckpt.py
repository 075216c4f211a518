"""GPU parity of the H-free path: sscan_fwd_ckpt keeps the state entering every 32-step
block instead of H, and sscan_bwd_ckpt recomputes each tile's states from those boundary
states.  Checked against the fp64 oracle (1e-4 for fp32, 2e-2 for y with bf16 I/O), the
boundary states against the oracle's H, and the gradients bitwise against sscan_bwd on the
forward's own H (the recomputation repeats the forward's arithmetic exactly)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import TOL_F32, announce, assert_close, to_dev, tol_for

pytestmark = pytest.mark.gpu

sscan = pytest.importorskip("selective_state_space_sscan_amd")
from selective_state_space_sscan_amd import (Plan, SScanError, selective_scan, sscan_bwd, sscan_bwd_ckpt,  # noqa: E402
                                             sscan_fwd, sscan_fwd_ckpt, sscan_mamba_bwd)

CK = 32
GR = ["gx", "gdelta", "gb", "gc", "gA", "gh0"]


def case(B, T, D, DS, io, seed, h0=True, dhT=True):
    w = workloads.custom(B, T, D, DS, io=io, seed=seed, h0_std=0.3 if h0 else 0.0, delta_mu=-1.0, with_dy=True,
                         with_dhT=dhT)
    return workloads.make_inputs(w)


CASES = [
    # B, T, D, DS, io, h0, dhT, fwd plan (lanes, chunks), bwd plan (lanes, chunks)
    (1, 1, 3, 8, "f32", True, True, (0, 0), (0, 0)),
    (2, 31, 17, 16, "f32", True, True, (0, 0), (0, 0)),
    (2, 33, 40, 16, "f32", False, True, (8, 1), (16, 1)),
    (2, 100, 65, 16, "f32", True, False, (8, 3), (16, 2)),
    (3, 257, 70, 8, "f32", True, True, (0, 0), (8, 3)),
    (2, 300, 40, 16, "bf16", True, True, (16, 2), (8, 2)),
    (1, 1000, 33, 16, "f32", True, True, (4, 5), (16, 5)),
]


@pytest.mark.parametrize("B,T,D,DS,io,h0,dhT,fplan,bplan", CASES)
def test_ckpt_forward_backward(gpu, B, T, D, DS, io, h0, dhT, fplan, bplan):
    announce(f"ckpt B={B} T={T} D={D} DS={DS} io={io} h0={h0} dhT={dhT} fwd plan={fplan} bwd plan={bplan}")
    inp = case(B, T, D, DS, io, seed=900 + B + T + D + DS, h0=h0, dhT=dhT)
    g = to_dev(inp, gpu)
    y, hT, hck = sscan_fwd_ckpt(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], plan=Plan(*fplan))
    grads = sscan_bwd_ckpt(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], hck, g["dhT"], plan=Plan(*bplan))
    torch.cuda.synchronize()
    yr, hTr, Hr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], return_H=True)
    assert tuple(hck.shape) == (B, (T + CK - 1) // CK, D, DS)
    h0r = np.zeros((B, D, DS)) if inp["h0"] is None else inp["h0"].double().numpy()
    ckr = np.stack([h0r] + [Hr[:, k * CK - 1] for k in range(1, hck.shape[1])], axis=1)
    assert_close("y", y, yr, tol_for(io))
    assert_close("hT", hT, hTr, TOL_F32)
    assert_close("hck", hck, ckr, TOL_F32)
    ref = oracle.bwd(inp["dy"], inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], inp["dhT"])
    for name, a, r in zip(GR, grads, ref):
        assert_close(name, a, r, TOL_F32)


@pytest.mark.parametrize("lanes,chunks", [(16, 1), (16, 3), (8, 2)])
def test_ckpt_gradients_equal_the_H_path_bitwise(gpu, lanes, chunks):
    B, T, D, DS = 2, 200, 48, 16
    announce(f"ckpt bitwise vs H path, bwd plan ({lanes},{chunks})")
    inp = case(B, T, D, DS, "f32", seed=931)
    g = to_dev(inp, gpu)
    one = Plan(8, 1, "lanes")  # single-chunk forwards in one layout: the same states and y whether kept or not
    y1, hT1, H = sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], return_H=True, plan=one)
    y2, hT2, hck = sscan_fwd_ckpt(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], plan=one)
    gH = sscan_bwd(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], H, g["dhT"], plan=Plan(lanes, chunks))
    gK = sscan_bwd_ckpt(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], hck, g["dhT"], plan=Plan(lanes, chunks))
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(hT1, hT2)
    assert torch.equal(hck[:, 1:], H[:, CK - 1::CK][:, : hck.shape[1] - 1])
    for name, a, b in zip(GR, gH, gK):
        assert torch.equal(a, b), name


def test_ckpt_mamba_wrapper(gpu):
    B, T, D, DS = 2, 150, 37, 16
    announce("ckpt with the Mamba-style wrapper")
    w = workloads.custom(B, T, D, DS, seed=944, h0_std=0.3, delta_mu=-1.0, with_dy=True, with_dhT=True)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    y, hT, hck = sscan_fwd_ckpt(g["x"], g["delta_raw"], g["A_log"], g["b"], g["c"], g["h0"], mamba=True,
                                Dskip=g["Dskip"])
    grads = sscan_bwd_ckpt(g["dy"], g["x"], g["delta_raw"], g["A_log"], g["b"], g["c"], hck, g["dhT"], mamba=True,
                           Dskip=g["Dskip"])
    torch.cuda.synchronize()
    yr, hTr = oracle.mamba_fwd(inp["x"], inp["delta_raw"], inp["A_log"], inp["b"], inp["c"], inp["Dskip"], inp["h0"])
    gx, gdr, gAl, gb, gc, gD, gh0 = oracle.mamba_bwd(inp["dy"], inp["x"], inp["delta_raw"], inp["A_log"], inp["b"],
                                                     inp["c"], inp["Dskip"], inp["h0"], inp["dhT"])
    assert_close("y", y, yr, TOL_F32)
    assert_close("hT", hT, hTr, TOL_F32)
    for name, a, r in zip(["gx", "gdelta_raw", "gb", "gc", "gA_log", "gh0", "gDskip"], grads,
                          [gx, gdr, gb, gc, gAl, gh0, gD]):
        assert_close(name, a, r, TOL_F32)


def test_ckpt_autograd(gpu):
    announce("selective_scan(ckpt=True) autograd")
    inp = case(2, 70, 33, 16, "f32", seed=951)
    g = to_dev(inp, gpu)
    leaves = {k: g[k].clone().requires_grad_(True) for k in ["x", "delta", "A", "b", "c", "h0"]}
    y, hT = selective_scan(*(leaves[k] for k in ["x", "delta", "A", "b", "c", "h0"]), ckpt=True)
    ((y * g["dy"]).sum() + (hT * g["dhT"]).sum()).backward()
    ref = oracle.bwd(inp["dy"], inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], inp["dhT"])
    for k, r in zip(["x", "delta", "b", "c", "A", "h0"], ref):
        assert_close("grad " + k, leaves[k].grad, r, TOL_F32)


def test_ckpt_backward_needs_eight_states(gpu):
    inp = case(1, 40, 8, 4, "f32", seed=960)
    g = to_dev(inp, gpu)
    y, hT, hck = sscan_fwd_ckpt(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"])
    with pytest.raises(SScanError):
        sscan_bwd_ckpt(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], hck, g["dhT"])


def test_ckpt_workload_size(gpu):
    announce("ckpt 8x2048x768x16 fp32 fwd+bwd")
    w = workloads.get("fwd_bwd_f32", with_dhT=True)
    inp = workloads.make_inputs(w)
    g = to_dev(inp, gpu)
    y, hT, hck = sscan_fwd_ckpt(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"])
    grads = sscan_bwd_ckpt(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], hck, g["dhT"])
    torch.cuda.synchronize()
    yr, hTr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"])
    assert_close("y", y, yr, TOL_F32)
    assert_close("hT", hT, hTr, TOL_F32)
    ref = oracle.bwd(inp["dy"], inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], inp["dhT"])
    for name, a, r in zip(GR, grads, ref):
        assert_close(name, a, r, TOL_F32)


@pytest.mark.parametrize("layout", ["lanes", "state_groups"])
@pytest.mark.parametrize("T", [31, 257, 100])
def test_ckpt_forward_writes_no_block_past_the_end(gpu, T, layout):
    """The tail tile's padded batches must not store boundary states: blocks past ceil(T/32)
    would land in the next batch row's blocks, or past the array."""
    B, D, DS = 3, 40, 16
    announce(f"ckpt guard region T={T} layout={layout}")
    inp = case(B, T, D, DS, "f32", seed=970 + T)
    g = to_dev(inp, gpu)
    nck = (T + CK - 1) // CK
    n = B * nck * D * DS
    guard = 4 * D * DS
    buf = torch.full((n + guard,), 12345.0, dtype=torch.float32, device=gpu)
    hck = buf[:n].view(B, nck, D, DS)
    sscan_fwd_ckpt(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], hck=hck, plan=Plan(0, 1, layout))
    torch.cuda.synchronize()
    assert bool((buf[n:] == 12345.0).all()), "a boundary state was written past the array"
    assert torch.equal(hck[:, 0], g["h0"])  # block 0 of every row is h0 itself


def test_ckpt_boundary_states_past_4gib(gpu):
    """Boundary states of one batch row spanning more than 4 GiB (D*DS = 2^22 states, 258
    blocks of 16 MiB): each tile addresses its blocks from a base of its own.  The last
    block must equal hT of a forward over the steps before it, and the gradients of the
    last 64 steps (dy zero elsewhere, no dhT) must equal those of the 64-step problem that
    starts from the boundary state there (the same sweep arithmetic on the same states)."""
    if torch.cuda.get_device_properties(gpu).total_memory < 96 * 2**30:
        pytest.skip("needs about 70 GiB of device memory")
    B, D, DS, T = 1, 1 << 18, 16, 8224  # 257 full blocks and the state entering the last one
    nck = (T + CK - 1) // CK
    assert nck * D * DS * 4 > 2**32
    announce(f"ckpt past 4 GiB: B={B} T={T} D={D} DS={DS} bf16 io, {nck} boundary blocks")
    gen = torch.Generator(device=gpu).manual_seed(4242)
    bf = torch.bfloat16
    x = torch.randn((B, T, D), generator=gen, device=gpu).to(bf)
    delta = torch.nn.functional.softplus(torch.randn((B, T, D), generator=gen, device=gpu) - 2.0).to(bf)
    b = torch.randn((B, T, DS), generator=gen, device=gpu).to(bf)
    c = torch.randn((B, T, DS), generator=gen, device=gpu).to(bf)
    A = -(torch.arange(1, DS + 1, device=gpu, dtype=torch.float32)[None, :]
          * (0.5 + torch.rand((D, DS), generator=gen, device=gpu)))
    y, hT, hck = sscan_fwd_ckpt(x, delta, A, b, c, None)
    t_cut = (nck - 1) * CK
    _, hT_cut = sscan_fwd(x[:, :t_cut], delta[:, :t_cut], A, b[:, :t_cut], c[:, :t_cut], None)
    torch.cuda.synchronize()
    assert torch.equal(hck[:, nck - 1], hT_cut), "last boundary block differs from the forward's state"
    del y, hT_cut
    # backward: dy only on the last 64 steps
    t0 = T - 64
    dy = torch.zeros((B, T, D), device=gpu, dtype=bf)
    dy[:, t0:] = torch.randn((B, 64, D), generator=gen, device=gpu).to(bf)
    gx, gd, gb, gc, _, _ = sscan_bwd_ckpt(dy, x, delta, A, b, c, hck, None)
    sl = slice(t0, T)
    _, _, hck2 = sscan_fwd_ckpt(x[:, sl], delta[:, sl], A, b[:, sl], c[:, sl], hck[:, t0 // CK].contiguous())
    gx2, gd2, gb2, gc2, _, _ = sscan_bwd_ckpt(dy[:, sl], x[:, sl], delta[:, sl], A, b[:, sl], c[:, sl], hck2, None)
    torch.cuda.synchronize()
    assert torch.equal(hck2[:, 1], hck[:, t0 // CK + 1])
    for name, a, r in (("gx", gx[:, sl], gx2), ("gdelta", gd[:, sl], gd2), ("gb", gb[:, sl], gb2),
                       ("gc", gc[:, sl], gc2)):
        assert torch.equal(a, r), f"{name} of the last 64 steps differs"
