"""Pins of the Mamba-3 SISO oracle (oracle/mamba3.py) against facts that do not come from the
oracle itself: closed forms of the trapezoid and Euler sums for a linear input, exact
exponential decay, the equivalence of RoPE on B/C with a complex-valued diagonal SSM,
RoPE's relative-position invariance, and the invariances of the norms.

Inputs are built so that the activations are known exactly: dt_raw = 0 with
dt_bias = log(expm1(dt)) gives dt; a_raw = log(expm1(a)) gives A = -a; trap_raw = 0, +800
and -800 give lambda = 1/2, 1 and 0 exactly; a zero norm weight with a bias row sets B or C
to that row exactly; z = 50 makes silu(z) = 50 exactly in f64.

MAMBA3_ORACLE_MUTANT (set by test_mamba3_mutants.py) points these pins at a copy of the
oracle with a planted mistake.
"""
import importlib.util
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load():
    path = os.environ.get("MAMBA3_ORACLE_MUTANT") or os.path.join(ROOT, "oracle", "mamba3.py")
    spec = importlib.util.spec_from_file_location("mamba3_under_test", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


o = _load()


def inv_softplus(v):
    return np.log(np.expm1(v))


class Seq:
    """One layer, one sequence, stepped T times through the oracle."""

    def __init__(self, nh=2, hd=3, ds=8, ng=1, na=0, a_floor=0.0, gate=False, rng=None):
        self.nh, self.hd, self.ds, self.ng, self.na, self.a_floor = nh, hd, ds, ng, na, a_floor
        rng = rng or np.random.default_rng(0)
        self.params = dict(dt_bias=np.zeros((1, nh)), b_norm_w=np.ones((1, ds)),
                           c_norm_w=np.ones((1, ds)), b_bias=np.zeros((1, nh, ds)),
                           c_bias=np.zeros((1, nh, ds)), D=np.zeros((1, nh)),
                           gate_w=np.ones((1, nh * hd)) if gate else None)
        self.h = np.zeros((1, 1, nh, hd, ds))
        self.k = np.zeros((1, 1, nh, ds))
        self.v = np.zeros((1, 1, nh, hd))
        self.ang = np.zeros((1, 1, nh, max(na, 1)))

    def row(self, z, x, B, C, dt_raw, a_raw, trap_raw, angles):
        parts = [np.broadcast_to(z, (self.nh * self.hd,)), np.broadcast_to(x, (self.nh * self.hd,)),
                 np.broadcast_to(B, (self.ng * self.ds,)), np.broadcast_to(C, (self.ng * self.ds,)),
                 np.broadcast_to(dt_raw, (self.nh,)), np.broadcast_to(a_raw, (self.nh,)),
                 np.broadcast_to(trap_raw, (self.nh,)), np.broadcast_to(angles, (self.na,))]
        r = np.concatenate([np.asarray(p, np.float64).ravel() for p in parts])
        assert r.size == o.proj_width(self.nh * self.hd, self.ng, self.ds, self.nh, self.na)
        return r

    def step(self, row):
        out, self.h, self.k, self.v, self.ang = o.siso_step(
            row[None, None], self.params, self.h, self.k, self.v, self.ang, nheads=self.nh,
            headdim=self.hd, d_state=self.ds, ngroups=self.ng, n_angles=self.na,
            a_floor=self.a_floor)
        return out[0, 0]


def fixed_bc(seq, b_row, c_row):
    """B and C set exactly to the given [nh, ds] rows: zero norm weights, bias rows."""
    seq.params["b_norm_w"][:] = 0.0
    seq.params["c_norm_w"][:] = 0.0
    seq.params["b_bias"][0] = b_row
    seq.params["c_bias"][0] = c_row


@pytest.mark.parametrize("trap_raw,expect", [
    (0.0, "trapezoid"),   # lambda = 1/2: exact for a linear input
    (800.0, "right"),     # lambda = 1: Euler, the right-endpoint sum
    (-800.0, "left"),     # lambda = 0: the left-endpoint sum
])
def test_linear_input_sums_closed_form(trap_raw, expect):
    """With A -> 0 the state is the quadrature of x over the steps. For x_t = a + b t
    (t = 0 .. T) the trapezoid rule is exact, dt T (x_0 + x_T) / 2; the right- and
    left-endpoint sums are dt (T a + b T (T + 1) / 2) and dt (T a + b T (T - 1) / 2)."""
    nh, hd, ds, T, dt = 2, 3, 4, 7, 0.37
    s = Seq(nh, hd, ds)
    s.params["dt_bias"][:] = inv_softplus(dt)
    fixed_bc(s, np.ones((nh, ds)), np.tile(np.eye(ds)[1], (nh, 1)))
    rng = np.random.default_rng(1)
    a = rng.normal(size=(nh, hd))
    b = rng.normal(size=(nh, hd))
    # the state before step 1 carries x_0 and B in the K/V states
    s.k[0, 0] = 1.0
    s.v[0, 0] = a
    for t in range(1, T + 1):
        out = s.step(s.row(50.0, (a + b * t).ravel(), 0.0, 0.0, 0.0, -60.0, trap_raw, []))
    sums = {"trapezoid": dt * T * (a + (a + b * T)) / 2,
            "right": dt * (T * a + b * T * (T + 1) / 2),
            "left": dt * (T * a + b * T * (T - 1) / 2)}
    want = sums[expect]
    np.testing.assert_allclose(s.h[0, 0][..., 2], want, rtol=1e-12, atol=1e-12)
    # the readout sees state component 1 (C = e_1), gated by silu(50) = 50, no D skip
    np.testing.assert_allclose(out.reshape(nh, hd), 50.0 * want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("a_raw_of,a_floor,decay", [
    (lambda: inv_softplus(0.8), 0.0, 0.8),
    (lambda: -60.0, 0.3, 0.3),  # softplus(-60) ~ 1e-26 is floored
])
def test_zero_input_decays_exactly(a_raw_of, a_floor, decay):
    """With x = 0 and no carried input the state only decays: h_T = exp(-T dt a) h_0."""
    nh, hd, ds, T, dt = 2, 3, 4, 5, 0.21
    s = Seq(nh, hd, ds, a_floor=a_floor)
    s.params["dt_bias"][:] = inv_softplus(dt)
    fixed_bc(s, np.zeros((nh, ds)), np.tile(np.eye(ds)[3], (nh, 1)))
    h0 = np.random.default_rng(2).normal(size=(nh, hd, ds))
    s.h[0, 0] = h0
    for _ in range(T):
        out = s.step(s.row(50.0, 0.0, 0.0, 0.0, 0.0, a_raw_of(), 0.0, []))
    want = np.exp(-T * dt * decay) * h0
    np.testing.assert_allclose(s.h[0, 0], want, rtol=1e-12, atol=0)
    np.testing.assert_allclose(out.reshape(nh, hd), 50.0 * want[..., 3], rtol=1e-12, atol=0)


def ode_error(trap_raw, dt, a=0.9, omega=2.0, horizon=2.0):
    """|h_T - h(horizon)| for h' = -a h + x(t), x(t) = cos(omega t), h(0) = 0, stepped with
    step size dt; the exact solution is (a cos wt + w sin wt - a e^{-at}) / (a^2 + w^2)."""
    nh, hd, ds = 1, 1, 2
    s = Seq(nh, hd, ds)
    s.params["dt_bias"][:] = inv_softplus(dt)
    fixed_bc(s, np.ones((nh, ds)), np.zeros((nh, ds)))
    s.k[0, 0] = 1.0
    s.v[0, 0] = 1.0  # x(0)
    T = int(round(horizon / dt))
    for t in range(1, T + 1):
        s.step(s.row(0.0, np.cos(omega * t * dt), 0.0, 0.0, 0.0, inv_softplus(a), trap_raw, []))
    exact = (a * np.cos(omega * horizon) + omega * np.sin(omega * horizon)
             - a * np.exp(-a * horizon)) / (a * a + omega * omega)
    return abs(s.h[0, 0, 0, 0, 0] - exact)


@pytest.mark.parametrize("trap_raw,order", [(0.0, 2), (800.0, 1)])
def test_convergence_order_on_an_ode(trap_raw, order):
    """The exponential-trapezoidal rule (lambda = 1/2) is second-order accurate on
    h' = A h + B x(t); the exponential-Euler end (lambda = 1) is first order. Halving the
    step divides the error at a fixed time by 4 and 2 respectively."""
    e1, e2 = ode_error(trap_raw, 0.02), ode_error(trap_raw, 0.01)
    assert abs(np.log2(e1 / e2) - order) < 0.1, (e1, e2)


def test_skip_term_from_zero_state():
    """From zero states with B = 0 the readout is the skip alone: out = silu(z) D x."""
    nh, hd, ds = 3, 4, 6
    s = Seq(nh, hd, ds)
    D = np.array([0.5, -1.25, 2.0])
    s.params["D"][0] = D
    fixed_bc(s, np.zeros((nh, ds)), np.ones((nh, ds)))
    x = np.random.default_rng(3).normal(size=(nh, hd))
    out = s.step(s.row(50.0, x.ravel(), 0.0, 0.0, 0.0, 0.0, 0.0, []))
    np.testing.assert_allclose(out.reshape(nh, hd), 50.0 * D[:, None] * x, rtol=1e-14, atol=0)


def rand_inputs(rng, seq, T, b_scale=1.0):
    rows = []
    for _ in range(T):
        rows.append(seq.row(rng.normal(size=seq.nh * seq.hd), rng.normal(size=seq.nh * seq.hd),
                            b_scale * rng.normal(size=seq.ng * seq.ds),
                            b_scale * rng.normal(size=seq.ng * seq.ds), rng.normal(size=seq.nh) * 0.5,
                            rng.normal(size=seq.nh), rng.normal(size=seq.nh), rng.normal(size=seq.na)))
    return rows


def random_params(seq, rng):
    seq.params["dt_bias"][0] = rng.normal(size=seq.nh) * 0.3
    seq.params["b_norm_w"][0] = 1.0 + 0.2 * rng.normal(size=seq.ds)
    seq.params["c_norm_w"][0] = 1.0 + 0.2 * rng.normal(size=seq.ds)
    seq.params["b_bias"][0] = 1.0 + 0.3 * rng.normal(size=(seq.nh, seq.ds))
    seq.params["c_bias"][0] = 1.0 + 0.3 * rng.normal(size=(seq.nh, seq.ds))
    seq.params["D"][0] = rng.normal(size=seq.nh)


@pytest.mark.parametrize("na", [4, 2, 0])
def test_rope_equals_complex_diagonal_ssm(na):
    """Rotating B and C by the running angle is a complex-valued diagonal SSM (Mamba-3's
    derivation): in rotated-back coordinates, pair i of the state is one complex number
    H_i with H_t = e^{-i phi_t} (alpha H_{t-1} + beta b_{t-1} x_{t-1}) + gamma b_t x_t and
    y_t = Re(sum_i conj(c_i) H_i) + D x, where phi_t = dt_t * omega_t is the angle step and
    b, c are the unrotated B and C pairs as complex numbers."""
    nh, hd, ds, T = 2, 3, 8, 9  # na = ds / 2 rotates every pair; fewer leaves the rest
    rng = np.random.default_rng(4)
    s = Seq(nh, hd, ds, na=na)
    random_params(s, rng)
    s.ang[0, 0, :, :na] = rng.normal(size=(nh, na))  # a nonzero starting angle
    # B, C raw entries are +-1 times a large scale: RMS-normalised they are the signs
    # (to ~1e-13), so the unrotated per-head B is sign * weight + bias, known exactly
    H = np.zeros((nh, hd, ds // 2), complex)
    b_prev = np.zeros((nh, ds // 2), complex)
    x_prev = np.zeros((nh, hd))
    for t in range(T):
        sb = rng.choice([-1.0, 1.0], size=ds)
        sc = rng.choice([-1.0, 1.0], size=ds)
        x = rng.normal(size=(nh, hd))
        dt_raw, a_raw, trap_raw = rng.normal(size=nh) * 0.5, rng.normal(size=nh), rng.normal(size=nh)
        omega = rng.normal(size=na)
        row = s.row(rng.normal(size=nh * hd) * 0 + 50.0, x.ravel(), 1e4 * sb, 1e4 * sc, dt_raw,
                    a_raw, trap_raw, omega)
        out = s.step(row)
        # the step's scalar coefficients (pinned by the closed-form tests above)
        dt, A, lam = o.activations(dt_raw, a_raw, trap_raw, s.params["dt_bias"][0], s.a_floor)
        alpha, beta, gamma = o.coefficients(dt, A, lam)
        Bu = sb * s.params["b_norm_w"][0] + s.params["b_bias"][0]  # [nh, ds]
        Cu = sc * s.params["c_norm_w"][0] + s.params["c_bias"][0]
        b = Bu[:, 0::2] + 1j * Bu[:, 1::2]
        c = Cu[:, 0::2] + 1j * Cu[:, 1::2]
        phi = np.zeros((nh, ds // 2))
        phi[:, :na] = dt[:, None] * omega[None, :]
        rot = np.exp(-1j * phi)[:, None, :]
        H = rot * (alpha[:, None, None] * H + beta[:, None, None] * x_prev[:, :, None] * b_prev[:, None, :]) \
            + gamma[:, None, None] * x[:, :, None] * b[:, None, :]
        y = np.real(np.einsum("hpi,hi->hp", H, np.conj(c))) + s.params["D"][0][:, None] * x
        np.testing.assert_allclose(out.reshape(nh, hd), 50.0 * y, rtol=1e-9, atol=1e-9)
        b_prev, x_prev = b, x


def test_angle_state_accumulates():
    """theta_T = theta_0 + sum_t dt_t omega_t, kept in the angle state."""
    nh, hd, ds, na, T, dt = 2, 2, 8, 3, 6, 0.45
    s = Seq(nh, hd, ds, na=na)
    s.params["dt_bias"][:] = inv_softplus(dt)
    th0 = np.random.default_rng(5).normal(size=(nh, na))
    s.ang[0, 0, :, :na] = th0
    omegas = np.random.default_rng(6).normal(size=(T, na))
    for t in range(T):
        s.step(s.row(0.0, 0.0, 1.0, 1.0, 0.0, 0.0, 0.0, omegas[t]))
    np.testing.assert_allclose(s.ang[0, 0, :, :na], th0 + dt * omegas.sum(0)[None, :], rtol=1e-12, atol=1e-12)


def test_rope_relative_position_invariance():
    """From zero SSM/K/V states, adding any constant to the starting angles leaves every
    output unchanged: the readout only sees angle differences."""
    nh, hd, ds, na, T = 2, 3, 8, 3, 6
    outs = []
    for shift in (0.0, 1.7):
        rng = np.random.default_rng(7)
        s = Seq(nh, hd, ds, na=na)
        random_params(s, rng)
        s.ang[0, 0, :, :na] = 0.3 + shift * np.arange(1, na + 1)
        outs.append([s.step(r) for r in rand_inputs(rng, s, T)])
    np.testing.assert_allclose(np.array(outs[1]), np.array(outs[0]), rtol=1e-10, atol=1e-10)
    # the rotation is not a no-op: other angle steps give other outputs
    rng = np.random.default_rng(7)
    s = Seq(nh, hd, ds, na=na)
    random_params(s, rng)
    s.ang[0, 0, :, :na] = 0.3
    rows = rand_inputs(rng, s, T)
    for r in rows:
        r[-na:] *= 2.0
    other = np.array([s.step(r) for r in rows])
    assert np.max(np.abs(other - np.array(outs[0]))) > 1e-3


def test_bc_norm_per_group_scale_invariance():
    """BC-norm normalises each group on its own: scaling one group's raw B and C by 3
    (at RMS ~100, where eps is negligible) leaves every output unchanged."""
    nh, hd, ds, ng, T = 4, 2, 6, 2, 4
    outs = []
    for scale in (1.0, 3.0):
        rng = np.random.default_rng(8)
        s = Seq(nh, hd, ds, ng=ng)
        random_params(s, rng)
        rows = rand_inputs(rng, s, T, b_scale=100.0)
        di, gs = nh * hd, ng * ds
        for r in rows:
            r[2 * di + ds:2 * di + gs] *= scale            # group 1 of B
            r[2 * di + gs + ds:2 * di + 2 * gs] *= scale   # group 1 of C
        outs.append(np.array([s.step(r) for r in rows]))
    np.testing.assert_allclose(outs[1], outs[0], rtol=1e-8, atol=1e-8)


def test_bc_norm_unit_rms():
    raw = np.random.default_rng(9).normal(size=(3, 16)) * 40.0
    out = o.bc_norm(raw, np.ones(16))
    np.testing.assert_allclose(np.sqrt(np.mean(out ** 2, axis=-1)), 1.0, rtol=1e-7)


def test_groups_map_to_consecutive_heads():
    """ngroups = 2, nheads = 4: heads 0, 1 read group 0 and heads 2, 3 group 1."""
    nh, hd, ds, ng = 4, 2, 4, 2
    res = []
    for bump in (0.0, 1.0):
        rng = np.random.default_rng(10)
        s = Seq(nh, hd, ds, ng=ng)
        random_params(s, rng)
        r = rand_inputs(rng, s, 1)[0]
        di, gs = nh * hd, ng * ds
        r[2 * di + ds:2 * di + gs] += bump * np.arange(ds)  # group 1 of B only
        res.append(s.step(r).reshape(nh, hd))
    np.testing.assert_array_equal(res[1][:2], res[0][:2])
    assert np.all(np.abs(res[1][2:] - res[0][2:]).max(axis=1) > 1e-6)


def test_gated_norm_is_per_head():
    """With the gate norm on, each head's headdim block has unit RMS (unit weights) and
    the sign of y * silu(z) (the same step with the plain silu gate)."""
    nh, hd, ds = 3, 8, 4
    outs = {}
    for gated in (True, False):
        rng = np.random.default_rng(11)
        s = Seq(nh, hd, ds, gate=gated)
        random_params(s, rng)
        s.params["D"][0] = [0.1, 1.0, 10.0]  # very different head scales
        outs[gated] = s.step(rand_inputs(rng, s, 1)[0]).reshape(nh, hd)
    g, plain = outs[True], outs[False]
    ms = np.mean(plain ** 2, axis=1)
    np.testing.assert_allclose(np.sqrt(np.mean(g ** 2, axis=1)), np.sqrt(ms / (ms + 1e-5)), rtol=1e-12)
    assert np.array_equal(np.sign(g), np.sign(plain))


def test_siso_step_pairs_subset_matches_full():
    """The sampled form (pairs=...) computes the same values as the full call."""
    L, B, nh, hd, ds, ng, na = 2, 3, 2, 2, 4, 1, 2
    rng = np.random.default_rng(12)
    W = o.proj_width(nh * hd, ng, ds, nh, na)
    proj = rng.normal(size=(L, B, W))
    params = dict(dt_bias=rng.normal(size=(L, nh)), b_norm_w=rng.normal(size=(L, ds)),
                  c_norm_w=rng.normal(size=(L, ds)), b_bias=rng.normal(size=(L, nh, ds)),
                  c_bias=rng.normal(size=(L, nh, ds)), D=rng.normal(size=(L, nh)),
                  gate_w=rng.normal(size=(L, nh * hd)))
    st = [rng.normal(size=(L, B, nh, hd, ds)), rng.normal(size=(L, B, nh, ds)),
          rng.normal(size=(L, B, nh, hd)), rng.normal(size=(L, B, nh, na))]
    kw = dict(nheads=nh, headdim=hd, d_state=ds, ngroups=ng, n_angles=na, a_floor=1e-4)
    full = o.siso_step(proj, params, *st, **kw)
    part = o.siso_step(proj, params, *st, pairs=[(1, 2), (0, 1)], **kw)
    for l, b in [(1, 2), (0, 1)]:
        for f, p in zip(full, part):
            np.testing.assert_array_equal(p[l, b], f[l, b])
    np.testing.assert_array_equal(part[1][0, 0], st[0][0, 0])  # untouched pairs copied through
