"""Mamba-3 SISO decode step, f64 CPU reference.

TEST INFRASTRUCTURE. Only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this module. It shares no code with the HIP library and never
imports it.

What it follows: the mamba3_siso inference.rs page (mamba-rs 0.2.1), the per-layer phase
list of its module doc and of ``step_layer_kernels``:

- F3: the 8-way split of the in_proj row, with softplus on dt, the floored softplus on A and
  the sigmoid on the trapezoid weight fused in;
- F4: BC-norm on B and C per group, the per-head bias (groups expanded to heads), the angle
  accumulation with its state and the rotation of B/C pairs;
- F5: alpha, beta, gamma from dt, A and the trapezoid weight;
- F6: the trapezoidal state update, which also uses the K state (the previous rotated B) and
  the V state (the previous x), then the readout and the D skip;
- F7: the output gate, either RMSNorm-gated per head or a plain silu gate.

The CUDA bodies of these kernels are not on the page. Each function states the reading it
takes of its phase; the readings are chosen to be the plainest ones that the page's buffer
shapes and argument lists support.

Everything is float64 numpy; inputs are converted on entry, so f32 inputs are read exactly.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-5  # the page's RMSNorm epsilon; BC-norm and the gated norm take no epsilon argument


def softplus(v):
    return np.logaddexp(0.0, v)


def sigmoid(v):
    return 0.5 * (1.0 + np.tanh(0.5 * v))  # no overflow for large |v|


def silu(v):
    return v * sigmoid(v)


def proj_width(d_inner, ngroups, d_state, nheads, n_angles):
    """Width of one in_proj row: z | x | B | C | dt | A | trap | angles (the order of
    m3_split's outputs on the page)."""
    return 2 * d_inner + 2 * ngroups * d_state + 3 * nheads + n_angles


def split(row, nheads, headdim, d_state, ngroups, n_angles):
    """F3 split of one in_proj row into its eight pieces (no arithmetic yet)."""
    di = nheads * headdim
    gs = ngroups * d_state
    o = 0
    parts = {}
    for name, width in (("z", di), ("x", di), ("B", gs), ("C", gs), ("dt", nheads),
                        ("A", nheads), ("trap", nheads), ("angles", n_angles)):
        parts[name] = row[o:o + width]
        o += width
    parts["z"] = parts["z"].reshape(nheads, headdim)
    parts["x"] = parts["x"].reshape(nheads, headdim)
    parts["B"] = parts["B"].reshape(ngroups, d_state)
    parts["C"] = parts["C"].reshape(ngroups, d_state)
    return parts


def activations(dt_raw, a_raw, trap_raw, dt_bias, a_floor):
    """F3's fused activations, per head.

    dt = softplus(dt_raw + dt_bias); A = -max(softplus(a_raw), a_floor) (the floor keeps
    every head decaying at least a little); lambda = sigmoid(trap_raw), the trapezoid
    weight in [0, 1]."""
    dt = softplus(dt_raw + dt_bias)
    A = -np.maximum(softplus(a_raw), a_floor)
    lam = sigmoid(trap_raw)
    return dt, A, lam


def bc_norm(raw, weight):
    """F4 BC-norm: RMSNorm of each group's d_state vector, times a [d_state] weight."""
    ms = np.mean(raw * raw, axis=-1, keepdims=True)
    return raw / np.sqrt(ms + EPS) * weight


def expand_groups(normed, bias, nheads):
    """F4 bias add: head h takes group h // (nheads / ngroups) (consecutive heads share a
    group) and adds its own [d_state] bias row."""
    ngroups = normed.shape[0]
    per = nheads // ngroups
    return normed[np.arange(nheads) // per] + bias


def accumulate_angles(angle_state, angles_raw, dt):
    """F4 angle step: theta[h, i] = angle_state[h, i] + dt[h] * angles_raw[i] (an inclusive
    running sum of dt-scaled angles). The returned theta is also the new angle state."""
    return angle_state + dt[:, None] * angles_raw[None, :]


def rope(v, theta):
    """F4 rotation: pair i = (v[2i], v[2i+1]) is turned by theta[i], for i < n_angles;
    the remaining components pass through."""
    out = v.copy()
    na = theta.shape[-1]
    if na == 0:
        return out
    a, b = v[..., 0:2 * na:2], v[..., 1:2 * na:2]
    c, s = np.cos(theta), np.sin(theta)
    out[..., 0:2 * na:2] = a * c - b * s
    out[..., 1:2 * na:2] = a * s + b * c
    return out


def coefficients(dt, A, lam):
    """F5: alpha = exp(dt * A), beta = (1 - lambda) * dt * alpha, gamma = lambda * dt.

    This is the exponential-trapezoidal rule of Mamba-3: the input integral over the step
    is weighted (1 - lambda) at its old end (carried by the decay alpha) and lambda at its
    new end; lambda = 1 is the Euler update of Mamba-1/2, lambda = 1/2 the trapezoid."""
    alpha = np.exp(dt * A)
    return alpha, (1.0 - lam) * dt * alpha, lam * dt


def state_update(h, k_prev, v_prev, k, x, alpha, beta, gamma):
    """F6: h[p, n] <- alpha h[p, n] + beta v_prev[p] k_prev[n] + gamma x[p] k[n], per head."""
    return (alpha[:, None, None] * h
            + beta[:, None, None] * v_prev[:, :, None] * k_prev[:, None, :]
            + gamma[:, None, None] * x[:, :, None] * k[:, None, :])


def readout(h, q, x, D):
    """F6 readout: y[p] = sum_n q[n] h[p, n] + D x[p], per head."""
    return np.einsum("hpn,hn->hp", h, q) + D[:, None] * x


def gate(y, z, gate_weight):
    """F7: g = y * silu(z). With a gate-norm weight (the page's outproj-norm option) each
    head's headdim block is RMS-normalised and scaled by the weight; without one, g is the
    output."""
    g = y * silu(z)
    if gate_weight is None:
        return g
    ms = np.mean(g * g, axis=-1, keepdims=True)
    return g / np.sqrt(ms + EPS) * gate_weight.reshape(g.shape)


def step_one(row, p, h, k_state, v_state, angle_state, nheads, headdim, d_state, ngroups,
             n_angles, a_floor):
    """One (layer, sequence) of the step. p holds that layer's parameters; the four states
    are that (layer, sequence)'s slices. Returns (out [d_inner], h, k, v, angle)."""
    s = split(row, nheads, headdim, d_state, ngroups, n_angles)
    dt, A, lam = activations(s["dt"], s["A"], s["trap"], p["dt_bias"], a_floor)
    Bh = expand_groups(bc_norm(s["B"], p["b_norm_w"]), p["b_bias"], nheads)
    Ch = expand_groups(bc_norm(s["C"], p["c_norm_w"]), p["c_bias"], nheads)
    theta = accumulate_angles(angle_state, s["angles"], dt)
    k, q = rope(Bh, theta), rope(Ch, theta)
    alpha, beta, gamma = coefficients(dt, A, lam)
    h_new = state_update(h, k_state, v_state, k, s["x"], alpha, beta, gamma)
    y = readout(h_new, q, s["x"], p["D"])
    out = gate(y, s["z"], p.get("gate_w"))
    return out.reshape(-1), h_new, k, s["x"].copy(), theta


def siso_step(proj, params, ssm_state, k_state, v_state, angle_state, *, nheads, headdim,
              d_state, ngroups, n_angles, a_floor, pairs=None):
    """The whole step for L layers and B sequences (every layer reads its own in_proj row;
    layers are independent here, as in a decode step given each layer's row).

    proj [L, B, W] with W = proj_width(...); params: dict of per-layer arrays with a leading
    L axis: dt_bias [L, nh], b_norm_w / c_norm_w [L, ds], b_bias / c_bias [L, nh, ds],
    D [L, nh], and gate_w [L, nh * hd] or None. States: ssm [L, B, nh, hd, ds],
    k [L, B, nh, ds], v [L, B, nh, hd], angle [L, B, nh, max(na, 1)] (only the first na
    angles are used).

    Returns out [L, B, nh * hd] and the four new states (new arrays). With ``pairs`` (a
    list of (l, b)) only those are computed; the rest of out is NaN and the rest of the
    states are copied through."""
    proj = np.asarray(proj, np.float64)
    L, B = proj.shape[:2]
    h_all = np.array(ssm_state, np.float64)
    k_all = np.array(k_state, np.float64)
    v_all = np.array(v_state, np.float64)
    a_all = np.array(angle_state, np.float64)
    out = np.full((L, B, nheads * headdim), np.nan)
    todo = pairs if pairs is not None else [(l, b) for l in range(L) for b in range(B)]
    for l, b in todo:
        p = {k: (None if v is None else np.asarray(v[l], np.float64)) for k, v in params.items()}
        o, h, k, v, th = step_one(proj[l, b], p, h_all[l, b], k_all[l, b], v_all[l, b],
                                  a_all[l, b, :, :n_angles], nheads, headdim, d_state, ngroups,
                                  n_angles, a_floor)
        out[l, b] = o
        h_all[l, b], k_all[l, b], v_all[l, b] = h, k, v
        a_all[l, b, :, :n_angles] = th
    return out, h_all, k_all, v_all, a_all
