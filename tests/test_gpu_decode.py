"""GPU parity of the one-token decode step (sscan_decode) against the fp64 oracle.

A decode step is the forward recurrence applied to one token with the state kept in
device memory, so its reference is the oracle's forward with T = 1 and h0 = the state;
a chain of decode steps must reproduce the oracle's forward over the whole sequence.
Tolerances as for the forward: 1e-4 (fp32 I/O), 2e-2 (bf16 I/O, fp32 state)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import TOL_F32, announce, assert_close, tol_for

pytestmark = pytest.mark.gpu

sscan = pytest.importorskip("selective_state_space_sscan_amd")
from selective_state_space_sscan_amd import sscan_decode  # noqa: E402

DECODE = [
    # B, D, DS, io
    (1, 1, 1, "f32"),
    (3, 37, 16, "f32"),
    (2, 100, 8, "bf16"),
    (5, 33, 4, "f32"),
    (4, 17, 2, "bf16"),
    (2, 300, 1, "f32"),
    (16, 1024, 16, "f32"),
    (16, 1024, 16, "bf16"),
]


def one_step(B, D, DS, io, seed):
    w = workloads.custom(B, 1, D, DS, io=io, seed=seed, h0_std=0.5, delta_mu=-1.0)
    return workloads.make_inputs(w)


@pytest.mark.parametrize("B,D,DS,io", DECODE)
@pytest.mark.parametrize("inplace", [False, True])
def test_decode_matches_one_step_oracle(gpu, B, D, DS, io, inplace):
    announce(f"decode B={B} D={D} DS={DS} io={io} inplace={inplace}")
    inp = one_step(B, D, DS, io, seed=B * 100 + D + DS)
    g = {k: (None if v is None else v.to(gpu)) for k, v in inp.items()}
    state = g["h0"].clone()
    y, s1 = sscan_decode(g["x"][:, 0], g["delta"][:, 0], g["A"], g["b"][:, 0], g["c"][:, 0], state, inplace=inplace)
    torch.cuda.synchronize()
    yr, hr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"])
    assert tuple(y.shape) == (B, D) and y.dtype == g["x"].dtype
    assert_close("y", y, yr[:, 0], tol_for(io))
    assert_close("state", s1, hr, TOL_F32)
    if inplace:
        assert s1.data_ptr() == state.data_ptr()
    else:
        assert torch.equal(state, g["h0"])  # the input state is left alone


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_chain_reproduces_the_forward(gpu, io):
    B, T, D, DS = 3, 48, 70, 16
    announce(f"decode chain B={B} T={T} D={D} DS={DS} io={io}")
    w = workloads.custom(B, T, D, DS, io=io, seed=77, h0_std=0.3, delta_mu=-1.0)
    inp = workloads.make_inputs(w)
    g = {k: (None if v is None else v.to(gpu)) for k, v in inp.items()}
    state = g["h0"].clone()
    ys = []
    for t in range(T):
        # alternate in-place and out-of-place updates: both must carry the state
        y, state = sscan_decode(g["x"][:, t], g["delta"][:, t], g["A"], g["b"][:, t], g["c"][:, t], state,
                                inplace=bool(t % 2))
        ys.append(y)
    torch.cuda.synchronize()
    yr, hr = oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"])
    assert_close("y", torch.stack(ys, dim=1), yr, tol_for(io))
    assert_close("state", state, hr, TOL_F32)


def test_decode_zero_delta_keeps_state_bitwise(gpu):
    announce("decode delta=0")
    inp = one_step(2, 40, 16, "f32", seed=5)
    g = {k: (None if v is None else v.to(gpu)) for k, v in inp.items()}
    zero = torch.zeros_like(g["delta"][:, 0])
    y, s1 = sscan_decode(g["x"][:, 0], zero, g["A"], g["b"][:, 0], g["c"][:, 0], g["h0"])
    torch.cuda.synchronize()
    assert torch.equal(s1, g["h0"])  # exp2(0) = 1 and a zero injection leave the state unchanged


def test_decode_empty_batch(gpu):
    announce("decode B=0")
    A = torch.zeros(8, 4, device=gpu)
    x = torch.zeros(0, 8, device=gpu)
    b = torch.zeros(0, 4, device=gpu)
    state = torch.zeros(0, 8, 4, device=gpu)
    y, s1 = sscan_decode(x, x, A, b, b, state)
    assert y.shape == (0, 8) and s1.shape == (0, 8, 4)


def test_decode_steps_replay_from_a_graph(gpu):
    """Decode steps captured in a HIP graph give, on every replay, exactly the eager result
    (the decode path launches only kernels: no memset or allocation is captured)."""
    announce("decode graph capture, 4 steps x 3 replays")
    inp = one_step(4, 96, 16, "f32", seed=11)
    g = {k: (None if v is None else v.to(gpu)) for k, v in inp.items()}
    x, dl, b, c = g["x"][:, 0], g["delta"][:, 0], g["b"][:, 0], g["c"][:, 0]
    steps = 4
    ref_state = g["h0"].clone()
    ref_y = torch.empty_like(x)
    for _ in range(steps):
        sscan_decode(x, dl, g["A"], b, c, ref_state, y=ref_y, inplace=True)
    torch.cuda.synchronize()
    state = torch.empty_like(g["h0"])
    y = torch.empty_like(x)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(device=gpu)
    cap.wait_stream(torch.cuda.current_stream(gpu))
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for _ in range(steps):
                sscan_decode(x, dl, g["A"], b, c, state, y=y, inplace=True)
    torch.cuda.current_stream(gpu).wait_stream(cap)
    torch.cuda.synchronize()
    for r in range(3):
        state.copy_(g["h0"])  # eager work between replays
        y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(state, ref_state), f"replay {r}: state differs"
        assert torch.equal(y, ref_y), f"replay {r}: y differs"
