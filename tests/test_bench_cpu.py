"""bench.py on the CPU: the multi-GPU refusal and the algorithmic byte counts the roofline
divides by (checked against sums written out per tensor, at the workloads' sizes)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_scan_bytes_130m_layer():
    # f32: u, dt, z in and y out per (t, d); B and C per t; state in and out; A_log, D, dt_bias
    B, T, D, N = 1, 2048, 1536, 16
    per_td = 4 * 4
    per_t = 2 * 4 * N
    state = 2 * 4 * N
    params = 4 * N + 4 + 4
    want = B * T * D * per_td + B * T * per_t + B * D * state + D * params
    assert bench.scan_bytes(4, B, T, D, N) == want


def test_decode_step_bytes_c2():
    L, B, D, N, K = 24, 64, 1536, 16, 4
    per_lbd = 4 * 4 + 2 * 4 * (N + K)    # x, dt, z, y; both states read and written
    per_lb = 2 * 4 * N                   # B and C rows
    per_ld = 4 * (K + 1) + 4 * N + 4 * 2  # taps + bias, A_log, D and dt_bias
    assert bench.decode_step_bytes(4, L, B, D, N, K) == L * (B * D * per_lbd + B * per_lb + D * per_ld)
    assert bench.decode_step_bytes(4, L, B, D, N, K) == 418824192


def test_m3_step_bytes_c5():
    s = W.C5
    heads = s.L * s.B * s.nheads
    state = 2 * 4 * s.headdim * s.d_state
    kva = 2 * 4 * (s.d_state + s.headdim + s.na)
    rows = s.L * s.B * (4 * s.width + 4 * s.d_inner)
    params = s.L * 4 * (s.nheads + 2 * s.d_state + 2 * s.nheads * s.d_state + s.nheads + s.d_inner)
    assert bench.m3_step_bytes(s) == heads * (state + kva) + rows + params == 2522903040


def test_valu_floor_constants():
    # the published fp32 vector peak (157.3 TFLOP/s) in fma lanes per second; 4 full-rate
    # slots plus a quarter-rate exp per element
    assert bench.VALU_SLOTS_PER_S == pytest.approx(157.3e12 / 2, rel=1e-3)
    assert bench.SCAN_SLOTS_PER_ELEMENT == 8
    floor_us = 8 * 4096 * 5120 * 16 * bench.SCAN_SLOTS_PER_ELEMENT / bench.VALU_SLOTS_PER_S * 1e6
    assert floor_us == pytest.approx(273.07, rel=1e-4)


def test_cpu_baseline_decode_small_shape():
    """The decode step's CPU oracle baseline on a small shape: whole steps within the budget,
    tokens/s/layer = L * B / (time of one step of L layers)."""
    s = W.DecodeShape("tiny", L=3, B=2, D=32, N=8, K=4)
    r = bench.cpu_baseline_decode(s, budget_s=0.5)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s/layer"
    assert r["value"] > 0 and r["cores"] >= 1 and r["seconds"] > 0
    assert "layers" in r["sample"] or "steps" in r["sample"]


def test_median_of_sampled_call_times():
    assert bench._median([3.0, 1.0, 2.0]) == 2.0
    assert bench._median([4.0, 1.0, 3.0, 2.0]) == 3.0
