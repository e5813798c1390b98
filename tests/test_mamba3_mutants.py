"""The Mamba-3 oracle pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle/mamba3.py and re-runs
tests/test_mamba3_oracle.py against that copy in a child process: at least one pin has to
fail. A mutation that no pin catches fails this test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mamba3.py")
PINS = os.path.join(ROOT, "tests", "test_mamba3_oracle.py")

MUTANTS = {
    "beta_uses_current_k": ("beta[:, None, None] * v_prev[:, :, None] * k_prev[:, None, :]",
                            "beta[:, None, None] * v_prev[:, :, None] * k[:, None, :]"),
    "beta_uses_current_x": ("beta[:, None, None] * v_prev[:, :, None] * k_prev[:, None, :]",
                            "beta[:, None, None] * x[:, :, None] * k_prev[:, None, :]"),
    "beta_gamma_swapped": ("return alpha, (1.0 - lam) * dt * alpha, lam * dt",
                           "return alpha, lam * dt * alpha, (1.0 - lam) * dt"),
    "beta_without_decay": ("return alpha, (1.0 - lam) * dt * alpha, lam * dt",
                           "return alpha, (1.0 - lam) * dt, lam * dt"),
    "decay_without_dt": ("alpha = np.exp(dt * A)", "alpha = np.exp(A)"),
    "A_sign": ("A = -np.maximum(softplus(a_raw), a_floor)", "A = np.maximum(softplus(a_raw), a_floor)"),
    "no_A_floor": ("A = -np.maximum(softplus(a_raw), a_floor)", "A = -softplus(a_raw)"),
    "no_dt_bias": ("    dt = softplus(dt_raw + dt_bias)\n", "    dt = softplus(dt_raw)\n"),
    "trap_weight_inverted": ("lam = sigmoid(trap_raw)", "lam = sigmoid(-trap_raw)"),
    "silu_sign": ("return v * sigmoid(v)", "return v * sigmoid(-v)"),
    "rope_on_k_only": ("k, q = rope(Bh, theta), rope(Ch, theta)", "k, q = rope(Bh, theta), Ch"),
    "rope_on_q_only": ("k, q = rope(Bh, theta), rope(Ch, theta)", "k, q = Bh, rope(Ch, theta)"),
    "rope_half_split_pairs": ("a, b = v[..., 0:2 * na:2], v[..., 1:2 * na:2]",
                              "a, b = v[..., 0:na], v[..., na:2 * na]"),
    "rope_not_a_rotation": ("out[..., 1:2 * na:2] = a * s + b * c", "out[..., 1:2 * na:2] = a * s - b * c"),
    "angle_not_accumulated": ("return angle_state + dt[:, None] * angles_raw[None, :]",
                              "return dt[:, None] * angles_raw[None, :]"),
    "angle_without_dt": ("return angle_state + dt[:, None] * angles_raw[None, :]",
                         "return angle_state + angles_raw[None, :]"),
    "no_bc_norm": ('Bh = expand_groups(bc_norm(s["B"], p["b_norm_w"]), p["b_bias"], nheads)',
                   'Bh = expand_groups(s["B"] * p["b_norm_w"], p["b_bias"], nheads)'),
    "bc_norm_over_all_groups": ("ms = np.mean(raw * raw, axis=-1, keepdims=True)", "ms = np.mean(raw * raw)"),
    "bc_bias_before_norm": ("return raw / np.sqrt(ms + EPS) * weight", "return raw / np.sqrt(ms + EPS) * weight + 0.5"),
    "groups_interleaved": ("return normed[np.arange(nheads) // per] + bias",
                           "return normed[np.arange(nheads) % ngroups] + bias"),
    "gate_norm_over_row": ("ms = np.mean(g * g, axis=-1, keepdims=True)", "ms = np.mean(g * g)"),
    "no_D_skip": ("+ D[:, None] * x", "+ 0.0 * x"),
    "readout_before_update": ('y = readout(h_new, q, s["x"], p["D"])', 'y = readout(h, q, s["x"], p["D"])'),
    "v_state_keeps_z": ('return out.reshape(-1), h_new, k, s["x"].copy(), theta',
                        'return out.reshape(-1), h_new, k, s["z"].copy(), theta'),
    "k_state_unrotated": ('return out.reshape(-1), h_new, k, s["x"].copy(), theta',
                          'return out.reshape(-1), h_new, Bh, s["x"].copy(), theta'),
    "split_order_B_C": ('for name, width in (("z", di), ("x", di), ("B", gs), ("C", gs),',
                        'for name, width in (("z", di), ("x", di), ("C", gs), ("B", gs),'),
}


def run_pins(path):
    env = dict(os.environ, MAMBA3_ORACLE_MUTANT=str(path))
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", PINS],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutant = tmp_path / "mamba3_mutant.py"
    mutant.write_text(src.replace(old, new))
    r = run_pins(mutant)
    assert r.returncode != 0, f"no pin caught mutant {name}:\n{r.stdout[-2000:]}"


def test_control_unmutated_copy_passes(tmp_path):
    """The same copy-and-rerun path with no mutation passes."""
    copy = tmp_path / "mamba3_copy.py"
    copy.write_text(open(SRC).read())
    r = run_pins(copy)
    assert r.returncode == 0, r.stdout[-2000:]
