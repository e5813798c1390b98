"""The oracle pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle/mamba_oracle.c (on the CPU), builds
it, and re-runs tests/test_oracle_pins.py against that build in a child process:
at least one pin has to fail. A mutation that no pin catches fails this test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mamba_oracle.c")

MUTANTS = {
    "A_sign": ("A[n] = -exp(A_log[(int64_t)d * N + n]);", "A[n] = exp(A_log[(int64_t)d * N + n]);"),
    "decay_without_delta": ("exp(delta * A[n]) * h[n]", "exp(A[n]) * h[n]"),
    "B_without_delta": ("delta * Bm[row * bc_row_stride + n] * ut", "Bm[row * bc_row_stride + n] * ut"),
    "readout_uses_B": ("yv += Cm[row * bc_row_stride + n] * h[n];", "yv += Bm[row * bc_row_stride + n] * h[n];"),
    "no_D_skip": ("yv += (D_skip ? D_skip[d] : 0.0) * ut;", "yv += 0.0 * ut;"),
    "gate_not_silu": ("y[row * D + d] = z ? yv * silu(z[row * z_row_stride + d]) : yv;",
                      "y[row * D + d] = z ? yv * z[row * z_row_stride + d] : yv;"),
    "no_dt_bias": ("double v = dt[row * D + d] + (dt_bias ? dt_bias[d] : 0.0);", "double v = dt[row * D + d];"),
    "softplus_sign": ("fmax(v, 0.0) + log1p(exp(-fabs(v)))", "fmax(v, 0.0) + log1p(exp(-v))"),
    "silu_sign": ("v / (1.0 + exp(-v))", "v / (1.0 + exp(v))"),
    "state_in_ignored": ("h[n] = ssm_state_in ? ssm_state_in[((int64_t)b * D + d) * N + n] : 0.0;", "h[n] = 0.0;"),
    "conv_taps_reversed": ("c += conv_w[(int64_t)d * K + k] * X[t + 1 + k];",
                           "c += conv_w[(int64_t)d * K + (K - 1 - k)] * X[t + 1 + k];"),
    "conv_window_off_by_one": ("c += conv_w[(int64_t)d * K + k] * X[t + 1 + k];",
                               "c += conv_w[(int64_t)d * K + k] * X[t + k];"),
    "conv_state_out_shifted": ("conv_state[((int64_t)b * D + d) * K + k] = X[T + k];",
                               "conv_state[((int64_t)b * D + d) * K + k] = X[T + k - 1];"),
    "conv_no_bias": ("double c = conv_b ? conv_b[d] : 0.0;\n      for (int k = 0; k < K; ++k) c += conv_w[(int64_t)d * K + k] * X[t + 1 + k];",
                     "double c = 0.0;\n      for (int k = 0; k < K; ++k) c += conv_w[(int64_t)d * K + k] * X[t + 1 + k];"),
    "step_B_without_delta": ("delta * Bm[(int64_t)b * bc_row_stride + n] * ut", "Bm[(int64_t)b * bc_row_stride + n] * ut"),
    "step_conv_no_shift": ("for (int k = 0; k + 1 < K; ++k) s[k] = s[k + 1];", "for (int k = 0; k + 1 < K; ++k) s[k] = s[k];"),
    "step_state_index": ("double* h = ssm_state + ((int64_t)b * D + d) * N;", "double* h = ssm_state + ((int64_t)d * B + b) * N;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                           "-ffp-contract=off", str(mutant_c), "-o", str(so), "-lm"])
    env = dict(os.environ, MAMBA_ORACLE_MUTANT_LIB=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"no oracle pin caught mutant {name}:\n{r.stdout[-2000:]}"


def test_control_unmutated_copy_passes(tmp_path):
    """The same build-and-rerun path with no mutation passes, so failures above come
    from the planted mistakes and not from the harness."""
    so = tmp_path / "libcontrol.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                           "-ffp-contract=off", SRC, "-o", str(so), "-lm"])
    env = dict(os.environ, MAMBA_ORACLE_MUTANT_LIB=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:]
