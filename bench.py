#!/usr/bin/env python3
"""Benchmark of the selective diagonal state-space scan on one MI355X.

One step = one pass of the whole hot path over one batch: the forward with the
per-step states H materialised, then the backward reverse sweep returning all six
gradients, on the fp32 workload B=8, T=2048, D=768, DS=16 (synthetic seeded
inputs, resident in HBM before timing starts; consecutive steps take three
copies of the inputs in turn, so no step starts with its inputs in the last-level
cache).  ``value`` is B*T*D elements per second of that step.  The JSON line
also carries:

* ``roofline`` for the entry point that dominates the step, timed live with HIP
  events on the stream the library launches on (torch's current stream), and the
  HBM traffic per launch from the committed rocprofv3 counter summary;
* ``cpu_baseline``: the fp64 CPU oracle timed on this host on the same workload
  (the value), plus one forward of each forward workload (``per_config``), the CPU
  model and the thread count;
* ``detail``: forward and backward times; the backward's HBM fraction on the method's
  bytes (every row of H read) and on the bytes the sweep as built moves;
* ``mamba`` and ``hfree``: the same step through the Mamba-style wrapper, and
  with boundary states every 32 steps in place of H;
* ``fwd_only``: forward-only throughput on the three forward workloads
  (fp32 8x1024x256x16; bf16 16x4096x1024x16; bf16 4x16384x2048x16 as 8 calls
  carrying hT -> h0), each with its ALU roofline fraction;
* ``decode``: one-token steps at 16x1024x16, replayed from a HIP graph.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-fwd-only]

The default warmup (80 steps, about 30 ms of work) runs past the first ~15 ms after a
start, in which the same kernels run 5-15% slower while the GPU's clocks settle, so the
timed steps measure the sustained rate.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks and unit counts.
HBM_PEAK_GBS = 8000.0
CUS, CLOCK_GHZ = 256, 2.4
# fp32 vector: 157.3 TFLOP/s = 128 fp32 lanes per CU per clock (256 CUs, 2.4 GHz), i.e.
# 78.6e12 single-lane fp32 ops/s; plain v_fma_f32 / v_mul_f32 reach that rate on gfx950.
FP32_LANES_PER_CU_CLK = 128
VALU_LANE_OPS = CUS * FP32_LANES_PER_CU_CLK * CLOCK_GHZ * 1e9  # 78.6e12 / s
# v_exp_f32 issues at a quarter of the fp32 lane rate: 32 lanes per CU per clock.
EXP_RATE = CUS * (FP32_LANES_PER_CU_CLK // 4) * CLOCK_GHZ * 1e9  # 19.7e12 / s
FWD_VALU_OPS_PER_STATE = 4  # delta*A, (delta x)*b, a*h+u, h*c+y
FWD_EXP_PER_STATE = 1


def alu_peak_states_per_s() -> float:
    """(step, channel, state) updates per second if VALU and v_exp_f32 issue back to back."""
    return 1.0 / (FWD_VALU_OPS_PER_STATE / VALU_LANE_OPS + FWD_EXP_PER_STATE / EXP_RATE)


PROFILE = os.path.join(ROOT, "profiles", "fwd_bwd_f32_B8_T2048_D768_DS16.md")
NSETS = 3  # input copies the step-type lines take in turn
KERNEL_SOURCES = ("fwd_kernel.h", "fwd.hip", "fwd_sg_kernel.h", "fwd_sg.hip", "bwd_kernel.h", "bwd.hip",
                  "device_common.h", "sscan_internal.h",
                  "sscan_api.cpp")


def kernel_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "selective_state_space_sscan_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(entry: str):
    """HBM bytes per launch of `entry` from the committed rocprofv3 counter summary, or None
    when the summary is missing or the kernel sources changed since it was taken."""
    try:
        with open(PROFILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    vals = {}
    for line in lines:
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != kernel_source_hash():
        return None
    v = vals.get(f"traffic_bytes_per_launch {entry}")
    return int(v) if v else None


def fwd_alg_bytes(B, T, D, DS, s, with_H=False):
    """Bytes the forward must move: x, delta in, y out; b, c in; A, h0 in, hT out; H out."""
    n = B * T * D
    byt = 3 * s * n + 2 * s * B * T * DS + 4 * D * DS + 2 * 4 * B * D * DS
    if with_H:
        byt += 4 * n * DS
    return byt


def bwd_alg_bytes(B, T, D, DS, s, h_read=1.0):
    """Bytes the backward must move: dy, x, delta in; H in; gx, gdelta out; b, c in; gb, gc out;
    A in, gA out; h0 in, gh0 out.  h_read: the fraction of H's rows read; the method reads every
    row (1.0, the algorithmic figure); the sweep as built with four states per lane reads every
    fourth row and forms the three after it from it (0.25)."""
    n = B * T * D
    return (3 * s * n + int(h_read * 4 * n * DS) + 2 * 4 * n + 2 * s * B * T * DS + 2 * 4 * B * T * DS
            + 2 * 4 * D * DS + 2 * 4 * B * D * DS)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=80)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fwd-only", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 3 times (to scale HBM byte counters)")
    ap.add_argument("--micro", action="store_true",
                    help="only measure the ceilings the kernels are compared against (v_exp_f32 and FMA rates, "
                         "the forward's per-state mix in registers, HBM read and write streams) and print them")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the scan runs on a single MI355X and the library has no multi-GPU "
              f"path (asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": src.numel() * 4, "bytes_written": dst.numel() * 4,
                          "launches": 3}))
        return 0

    if args.micro:
        print(json.dumps({"micro": micro_rates()}))
        return 0

    import workloads
    from selective_state_space_sscan_amd import sscan_bwd, sscan_bwd_workspace, sscan_fwd, sscan_fwd_workspace
    from selective_state_space_sscan_amd import sscan_plan_select

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = workloads.get("fwd_bwd_f32")
    B, T, D, DS = w.B, w.T, w.D, w.DS
    print(f"bench: {w.name} {w.note} on {torch.cuda.get_device_name(dev)}", file=sys.stderr, flush=True)
    inp = workloads.make_inputs(w)
    # Consecutive steps take different batches (NSETS copies of the inputs in turn), so no
    # step finds its inputs in the 256 MB last-level cache where the step before left them.
    sets = [{k: (None if v is None else v.to(dev)) for k, v in inp.items()} for _ in range(NSETS)]
    f32 = dict(dtype=torch.float32, device=dev)
    y = torch.empty((B, T, D), **f32)
    hT = torch.empty((B, D, DS), **f32)
    H = torch.empty((B, T, D, DS), **f32)
    outs = (torch.empty((B, T, D), **f32), torch.empty((B, T, D), **f32), torch.empty((B, T, DS), **f32),
            torch.empty((B, T, DS), **f32), torch.empty((D, DS), **f32), torch.empty((B, D, DS), **f32))
    ws_f = torch.empty(max(1, sscan_fwd_workspace(B, T, D, DS)), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(1, sscan_bwd_workspace(B, T, D, DS)), dtype=torch.uint8, device=dev)
    plan_f = sscan_plan_select(B, T, D, DS, with_H=True)
    plan_b = sscan_plan_select(B, T, D, DS, backward=True)

    def fwd(k):
        g = sets[k % NSETS]
        sscan_fwd(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], y=y, hT=hT, H=H, workspace=ws_f)

    def bwd(k):
        g = sets[k % NSETS]
        sscan_bwd(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], H, None, workspace=ws_b, out=outs)

    for k in range(args.warmup):
        fwd(k)
        bwd(k)
    torch.cuda.synchronize()

    K = args.steps
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        ev[k][0].record(stream)
        fwd(k)
        ev[k][1].record(stream)
        bwd(k)
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = np.array([ev[k][0].elapsed_time(ev[k][1]) for k in range(K)])
    bwd_ms = np.array([ev[k][1].elapsed_time(ev[k][2]) for k in range(K)])
    step_ms = ev[0][0].elapsed_time(ev[K - 1][2]) / K
    elems = B * T * D
    value = elems / (step_ms * 1e-3)

    fbytes = fwd_alg_bytes(B, T, D, DS, 4, with_H=True)
    bbytes = bwd_alg_bytes(B, T, D, DS, 4)
    bbytes_built = bwd_alg_bytes(B, T, D, DS, 4, h_read=0.25)
    f_avg, b_avg = float(fwd_ms.mean()), float(bwd_ms.mean())
    # The dominant entry point is timed as one launch: sscan_bwd enqueues the local pass of
    # its two-level sweep, the sweep and the kernel that adds its partial sums, back to back
    # on the same stream.
    if b_avg >= f_avg:
        dom, entry, dom_bytes, dom_ms = ("sscan_bwd (bwd_local_kernel + bwd_kernel sweep + bwd_reduce_kernel)",
                                         "sscan_bwd", bbytes, b_avg)
    else:
        kern = ("bc_pack_kernel + fwd_sg_kernel writing H through LDS" if plan_f.layout == "state_groups"
                else "fwd_kernel writing H")
        dom, entry, dom_bytes, dom_ms = f"sscan_fwd ({kern})", "sscan_fwd", fbytes, f_avg
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = committed_traffic(entry)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": dom,
                "alg_bytes_per_launch": int(dom_bytes), "avg_launch_ms": round(dom_ms, 5)}
    detail = {
        "fwd_ms": round(f_avg, 5), "bwd_ms": round(b_avg, 5),
        "fwd_elems_per_s": elems / (f_avg * 1e-3), "bwd_elems_per_s": elems / (b_avg * 1e-3),
        "fwd_hbm_frac": round(fbytes / (f_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "bwd_hbm_frac": round(bbytes / (b_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "bwd_alg_bytes": int(bbytes),
        "bwd_hbm_frac_as_built": round(bbytes_built / (b_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "bwd_bytes_as_built": int(bbytes_built),
        "plan_fwd": {"lanes": plan_f.lanes, "chunks": plan_f.chunks, "layout": plan_f.layout},
        "plan_bwd": {"lanes": plan_b.lanes, "chunks": plan_b.chunks},
        "wall_s_timed": round(wall, 4),
    }
    print(f"bench: step {step_ms:.4f} ms (fwd {f_avg:.4f}, bwd {b_avg:.4f})", file=sys.stderr, flush=True)

    mamba = None if args.no_fwd_only else bench_mamba(sets, y, hT, H, outs, B, T, D, args.warmup, max(10, K // 2))
    hfree = None if args.no_fwd_only else bench_hfree(sets, y, hT, outs, B, T, D, DS, args.warmup, max(10, K // 2))
    fwd_only = None if args.no_fwd_only else bench_fwd_only(dev, args.warmup, max(5, K // 5))
    decode = None if args.no_fwd_only else bench_decode(dev, args.warmup, max(5, K // 5))

    cpu = None
    if not args.no_cpu_baseline:
        del sets
        torch.cuda.empty_cache()
        cpu = cpu_baseline(inp, w)

    line = {
        "metric": "selective-scan fwd B*T*D/sec on 1 MI355X; % of HBM/VALU roofline; bwd B*T*D/sec",
        "value": value, "unit": "B*T*D elements/s (forward with H + backward, one step)",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": step_ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "fwd+bwd B=8 T=2048 D=768 DS=16 fp32, H materialised, 6 gradients",
                   "B": B, "T": T, "D": D, "DS": DS, "io": "f32"},
        "roofline": roofline, "cpu_baseline": cpu, "detail": detail, "hfree": hfree, "mamba": mamba,
        "fwd_only": fwd_only,
        "decode": decode,
    }
    print(json.dumps(line))
    return 0


def micro_rates():
    """Ceilings measured by the kernels of libsscan_micro.so (built with libsscan): per-CU-clock
    figures use 256 CUs at 2.4 GHz."""
    import ctypes

    path = os.path.join(ROOT, "selective_state_space_sscan_amd", "libsscan_micro.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with python -m selective_state_space_sscan_amd.build")
    lib = ctypes.CDLL(path)
    lib.sscan_micro_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.POINTER(ctypes.c_double)]
    lib.sscan_micro_rate.restype = ctypes.c_int

    def rate(which, waves, nbytes=0):
        r = ctypes.c_double()
        if lib.sscan_micro_rate(which, waves, nbytes, ctypes.byref(r)) != 0:
            raise RuntimeError(f"sscan_micro_rate({which}, {waves}, {nbytes}) failed")
        return r.value

    per_cu_clk = 256 * 2.4e9
    out = {"exp2_per_s": {w: rate(0, w) for w in (1, 2, 4, 8)},
           "fma_per_s": {w: rate(1, w) for w in (1, 2, 4, 8)},
           "mix_states_per_cu_clk": {f"K{k} W{w}": round(rate(which, w) / per_cu_clk, 2)
                                     for which, k in ((2, 1), (3, 2), (4, 4)) for w in (1, 2, 3, 4, 8)},
           "write_stream_GBps": rate(5, 1, 2 << 30) / 1e9,
           "write_stream_nontemporal_GBps": rate(7, 1, 2 << 30) / 1e9,
           "h_store_pattern_8x2048x768x16_GBps": rate(8, 1) / 1e9,
           "fwd_h_memory_pattern_8x2048x768x16_GBps": rate(9, 1) / 1e9,
           "fwd_h_memory_pattern_8x2048x768x16_cold_inputs_GBps": rate(10, 1) / 1e9,
           "read_stream_GBps": rate(6, 1, 2 << 30) / 1e9}
    # torch's own fill and copy kernels on 2 GiB, for comparison with the plain streams above
    import torch

    buf = torch.empty(1 << 29, dtype=torch.float32, device="cuda")
    src = torch.ones_like(buf)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    buf.fill_(1.0)
    buf.copy_(src)
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(10):
        buf.fill_(2.0)
    ev[1].record()
    for _ in range(10):
        buf.copy_(src)
    ev[2].record()
    torch.cuda.synchronize()
    out["torch_fill_GBps"] = buf.numel() * 4 / (ev[0].elapsed_time(ev[1]) / 10 * 1e-3) / 1e9
    out["torch_copy_GBps_read_plus_written"] = 2 * buf.numel() * 4 / (ev[1].elapsed_time(ev[2]) / 10 * 1e-3) / 1e9
    del buf, src
    for k, v in out.items():
        print(f"micro: {k}: {v}", file=sys.stderr, flush=True)
    return out


def time_fwd_bwd(fwd, bwd, warmup, reps):
    """Average forward and backward times of `reps` steps run back to back, as the main
    step is timed: events between the calls, one synchronisation after the last step (so
    the host's launch latency is not inside the events)."""
    import torch

    for k in range(warmup):
        fwd(k)
        bwd(k)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for k in range(reps):
        ev[k][0].record()
        fwd(k)
        ev[k][1].record()
        bwd(k)
        ev[k][2].record()
    torch.cuda.synchronize()
    f_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / reps
    b_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / reps
    return f_ms, b_ms


def bench_hfree(sets, y, hT, outs, B, T, D, DS, warmup, reps):
    """The H-free path on the same workload: the forward keeps the state entering every
    32-step block instead of H, the backward recomputes each tile's states from them."""
    import torch

    from selective_state_space_sscan_amd import sscan_bwd_ckpt, sscan_fwd_ckpt

    dev = sets[0]["x"].device
    hck = torch.empty((B, (T + 31) // 32, D, DS), dtype=torch.float32, device=dev)

    def fwd(k):
        g = sets[k % NSETS]
        sscan_fwd_ckpt(g["x"], g["delta"], g["A"], g["b"], g["c"], g["h0"], y=y, hT=hT, hck=hck)

    def bwd(k):
        g = sets[k % NSETS]
        sscan_bwd_ckpt(g["dy"], g["x"], g["delta"], g["A"], g["b"], g["c"], hck, None, out=outs)

    f_ms, b_ms = time_fwd_bwd(fwd, bwd, warmup, reps)
    print(f"bench: H-free fwd {f_ms:.4f} ms, bwd {b_ms:.4f} ms", file=sys.stderr, flush=True)
    return {"workload": f"fwd+bwd B={B} T={T} D={D} DS={DS} fp32 with boundary states every 32 steps instead of H "
                        "(1/32 of its memory); the backward recomputes each tile's states",
            "fwd_ms": f_ms, "bwd_ms": b_ms, "ms_per_step": f_ms + b_ms,
            "elems_per_s": B * T * D / ((f_ms + b_ms) * 1e-3),
            "state_bytes": hck.numel() * 4, "H_bytes": B * T * D * DS * 4}


def bench_mamba(sets, y, hT, H, outs, B, T, D, warmup, reps):
    """The Mamba-style wrapper (softplus step, A = -exp(A_log), skip term fused into the
    scan kernels) on the same workload and buffers: forward with H and backward."""
    import torch

    from selective_state_space_sscan_amd import sscan_mamba_bwd, sscan_mamba_bwd_workspace, sscan_mamba_fwd

    dev = sets[0]["x"].device
    ws_b = torch.empty(max(1, sscan_mamba_bwd_workspace(B, T, D, H.shape[-1])), dtype=torch.uint8, device=dev)
    gD = torch.empty((D,), dtype=torch.float32, device=dev)
    mouts = tuple(outs) + (gD,)

    def fwd(k):
        g = sets[k % NSETS]
        sscan_mamba_fwd(g["x"], g["delta_raw"], g["A_log"], g["b"], g["c"], g["Dskip"], g["h0"], y=y, hT=hT, H=H)

    def bwd(k):
        g = sets[k % NSETS]
        sscan_mamba_bwd(g["dy"], g["x"], g["delta_raw"], g["A_log"], g["b"], g["c"], g["Dskip"], g["h0"], H, None,
                        workspace=ws_b, out=mouts)

    f_ms, b_ms = time_fwd_bwd(fwd, bwd, warmup, reps)
    print(f"bench: mamba wrapper fwd {f_ms:.4f} ms, bwd {b_ms:.4f} ms", file=sys.stderr, flush=True)
    return {"workload": f"Mamba-style wrapper on B={B} T={T} D={D}: softplus(delta_raw), -exp(A_log), Dskip*x; "
                        "fwd writes H, bwd returns 7 gradients",
            "fwd_ms": f_ms, "bwd_ms": b_ms, "elems_per_s": B * T * D / ((f_ms + b_ms) * 1e-3)}


def bench_decode(dev, warmup, reps):
    """One-token decode steps on a resident state.  A run of consecutive in-place steps is
    captured once in a HIP graph and replayed, so the time per step is the GPU's (eager
    calls from Python are host-bound at this size); the eager per-call time is reported
    beside it."""
    import torch

    import workloads
    from selective_state_space_sscan_amd import sscan_decode

    out = {}
    B, D, DS = 16, 1024, 16
    for io in ("f32", "bf16"):
        w = workloads.custom(B, 1, D, DS, io=io, seed=9, h0_std=0.1)
        g = {k: (None if v is None else v.to(dev)) for k, v in workloads.make_inputs(w).items()}
        x, dl, b, c = g["x"][:, 0], g["delta"][:, 0], g["b"][:, 0], g["c"][:, 0]
        state = g["h0"].clone()
        y = torch.empty((B, D), dtype=x.dtype, device=dev)
        for _ in range(max(warmup, 3)):
            sscan_decode(x, dl, g["A"], b, c, state, y=y, inplace=True)
        torch.cuda.synchronize()
        n = max(1000, reps * 10)  # ~15 ms of host-bound calls: a steadier figure than 100
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            sscan_decode(x, dl, g["A"], b, c, state, y=y, inplace=True)
        e1.record()
        torch.cuda.synchronize()
        us_eager = e0.elapsed_time(e1) * 1e3 / n
        steps = 32
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(device=dev)
        cap.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                for _ in range(steps):
                    sscan_decode(x, dl, g["A"], b, c, state, y=y, inplace=True)
        torch.cuda.current_stream(dev).wait_stream(cap)
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        reps_g = max(10, reps)
        e0.record()
        for _ in range(reps_g):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps_g * steps)
        s = 2 if io == "bf16" else 4
        nbytes = B * D * DS * 8 + B * D * 3 * s + B * DS * 2 * s + D * DS * 4
        out[io] = {"workload": f"decode step B={B} D={D} DS={DS} {io} I/O, state fp32 in place",
                   "us_per_step": us, "us_per_step_eager_python": us_eager,
                   "tokens_per_s": B / (us * 1e-6), "gb_per_s": nbytes / (us * 1e-6) / 1e9}
        print(f"bench: decode {io}: {us:.2f} us/step in a graph, {us_eager:.2f} us/step eager",
              file=sys.stderr, flush=True)
    return out


def bench_fwd_only(dev, warmup, reps):
    """Forward-only rates on the three forward workloads, against the ALU roofline."""
    import torch

    import workloads
    from selective_state_space_sscan_amd import sscan_fwd, sscan_fwd_workspace, sscan_plan_select

    out = {}
    peak = alu_peak_states_per_s()
    # what bounds each workload, from the kernel traces and vector-ALU counters (profiles/)
    bound = {"fwd_f32": "latency: 3.4e7 state updates and 26 MB, run as two passes over 16 chunks of 64 steps "
                        "(local pass, full pass)",
             "fwd_bf16": "VALU issue: the SIMDs issue ~84% of cycles at ~5.8 instructions per state "
                         "(floor 5 without packed FP32)",
             "long_chunked_bf16": "VALU latency: one compute wave per SIMD, ~63% of SIMD cycles issuing"}
    for name in ("fwd_f32", "fwd_bf16", "long_chunked_bf16"):
        w = workloads.get(name)
        inp = workloads.make_inputs(w)
        dt = inp["x"].dtype
        s = 2 if dt == torch.bfloat16 else 4
        bounds = workloads.chunk_bounds(w.T, w.chunks)
        tc = bounds[0][1] - bounds[0][0]
        # rotate input copies so the 256 MB last-level cache cannot hold a small workload
        footprint = fwd_alg_bytes(w.B, w.T, w.D, w.DS, s)
        ncopy = max(1, min(16, int(512e6 // max(footprint, 1))))
        sets = []
        for _ in range(ncopy):
            sets.append({k: (None if v is None else v.to(dev)) for k, v in inp.items()})
        del inp
        y = torch.empty((w.B, w.T, w.D), dtype=dt, device=dev)
        hT = torch.empty((w.B, w.D, w.DS), dtype=torch.float32, device=dev)
        hbuf = torch.empty((w.B, w.D, w.DS), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, sscan_fwd_workspace(w.B, tc, w.D, w.DS, dt)), dtype=torch.uint8, device=dev)
        plan = sscan_plan_select(w.B, tc, w.D, w.DS, dt)

        def run(g):
            # consecutive calls carry the state; the two state buffers alternate so no
            # call's hT output aliases its h0 input
            h = g["h0"]
            for i, (t0, t1) in enumerate(bounds):
                sl = slice(t0, t1)
                dst = (hbuf, hT)[i % 2]
                sscan_fwd(g["x"][:, sl], g["delta"][:, sl], g["A"], g["b"][:, sl], g["c"][:, sl], h,
                          y=y[:, sl], hT=dst, workspace=ws)
                h = dst

        for i in range(warmup):
            run(sets[i % ncopy])
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        # time at least ~25 ms of work: ten calls of the small workload (~0.03 ms each) are
        # too short a window for a steady figure
        e0.record()
        for i in range(5):
            run(sets[i % ncopy])
        e1.record()
        torch.cuda.synchronize()
        n = max(reps, min(2000, int(25.0 / max(e0.elapsed_time(e1) / 5, 1e-3))))
        e0.record()
        for i in range(n):
            run(sets[i % ncopy])
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        elems = w.B * w.T * w.D
        states = elems * w.DS
        out[name] = {"workload": w.note, "calls": len(bounds), "timed_runs": n,
                     "plan": {"lanes": plan.lanes, "chunks": plan.chunks, "layout": plan.layout},
                     "ms": round(ms, 5), "elems_per_s": elems / (ms * 1e-3),
                     "alu_frac": round(states / (ms * 1e-3) / peak, 4),
                     "hbm_frac": round(fwd_alg_bytes(w.B, w.T, w.D, w.DS, s) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "bound": bound[name]}
        print(f"bench: fwd-only {name}: {ms:.4f} ms, {elems / (ms * 1e-3):.3e} elem/s", file=sys.stderr, flush=True)
        del sets
        torch.cuda.empty_cache()
    out["alu_peak_states_per_s"] = peak
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, w):
    """The fp64 oracle, as it stands, on this host: one forward + backward of the whole bench
    workload (the line's value), then one forward of each forward workload at full size (the
    long one as a single unchunked pass over all its steps), and the smallest one on one core."""
    import oracle
    import workloads

    n = oracle.default_threads()
    t0 = time.perf_counter()
    oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], nthreads=n)
    t1 = time.perf_counter()
    oracle.bwd(inp["dy"], inp["x"], inp["delta"], inp["A"], inp["b"], inp["c"], inp["h0"], None, nthreads=n)
    t2 = time.perf_counter()
    elems = w.B * w.T * w.D
    per = {f"{w.name}_fwd": {"s": round(t1 - t0, 4), "cores": n, "elems_per_s": elems / (t1 - t0)},
           f"{w.name}_bwd": {"s": round(t2 - t1, 4), "cores": n, "elems_per_s": elems / (t2 - t1)}}
    for name, threads in (("fwd_f32", n), ("fwd_f32", 1), ("fwd_bf16", n), ("long_chunked_bf16", n)):
        wl = workloads.get(name)
        x = workloads.make_inputs(wl)
        a = time.perf_counter()
        oracle.fwd(x["x"], x["delta"], x["A"], x["b"], x["c"], x["h0"], nthreads=threads)
        dt = time.perf_counter() - a
        del x
        key = f"{name}_fwd" + ("" if threads == n else f"_{threads}core")
        per[key] = {"s": round(dt, 4), "cores": threads, "elems_per_s": wl.elems / dt}
        print(f"bench: oracle {key}: {dt:.3f} s on {threads} cores", file=sys.stderr, flush=True)
    return {"value": elems / (t2 - t0), "unit": "B*T*D elements/s (forward + backward)", "cores": n, "kind": "oracle",
            "sample": f"the whole {w.B}x{w.T}x{w.D}x{w.DS} workload, one forward (no H) + one backward "
                      f"(which recomputes its states); fwd {t1 - t0:.3f} s, bwd {t2 - t1:.3f} s",
            "cpu_model": cpu_model(), "per_config": per}


if __name__ == "__main__":
    sys.exit(main())
