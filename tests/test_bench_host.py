"""Host-side checks of bench.py: the one-GPU contract and the byte and ALU figures its
roofline fields are built from (no GPU needed)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_forward_bytes_per_element():
    # fp32 I/O at 8x2048x768x16: x, delta read and y written (12 B), b and c (8 B per
    # (b, t, n), spread over D), A, h0, hT; with H another 64 B per element
    B, T, D, DS = 8, 2048, 768, 16
    n = B * T * D
    plain = bench.fwd_alg_bytes(B, T, D, DS, 4)
    with_h = bench.fwd_alg_bytes(B, T, D, DS, 4, with_H=True)
    assert with_h - plain == 64 * n
    assert plain == 12 * n + 8 * B * T * DS + 4 * D * DS + 8 * B * D * DS
    assert abs(with_h / 1e6 - 959.2) < 0.1


def test_backward_bytes_per_element():
    B, T, D, DS = 8, 2048, 768, 16
    n = B * T * D
    full = bench.bwd_alg_bytes(B, T, D, DS, 4, h_read=1.0)
    # dy, x, delta read (12), H read (64), gx, gdelta written (8); b, c read and gb, gc
    # written (16 B per (b, t, n)); A read, gA written; h0 read, gh0 written
    assert full == 84 * n + 16 * B * T * DS + 8 * D * DS + 8 * B * D * DS
    assert abs(full / 1e6 - 1062.0) < 0.1
    assert bench.bwd_alg_bytes(B, T, D, DS, 4) == full  # the method's bytes are the default
    # the sweep as built reads every fourth row of H
    got = bench.bwd_alg_bytes(B, T, D, DS, 4, h_read=0.25)
    assert full - got == 48 * n
    assert abs(got / 1e6 - 458.1) < 0.1
    # bf16 I/O halves only the three (B,T,D) inputs and b, c
    assert bench.bwd_alg_bytes(B, T, D, DS, 2, h_read=0.25) == got - 6 * n - 4 * B * T * DS


def test_alu_peak_from_unit_counts():
    # 256 CUs x 128 fp32 lanes x 2.4 GHz, exp at a quarter rate, 4 ops + 1 exp per state
    lane_ops = 256 * 128 * 2.4e9
    assert bench.VALU_LANE_OPS == pytest.approx(lane_ops)
    assert bench.alu_peak_states_per_s() == pytest.approx(1.0 / (4 / lane_ops + 1 / (lane_ops / 4)))
    assert bench.alu_peak_states_per_s() == pytest.approx(9.83e12, rel=1e-3)


def test_kernel_hash_covers_existing_sources():
    for f in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, "selective_state_space_sscan_amd", "csrc", f)), f
    assert len(bench.kernel_source_hash()) == 16
