"""Pins of the f64 oracle against facts that do not come from the oracle itself:
hand-worked values, closed forms, brute force through a different formula,
library routines for special cases, and invariants of the method.

Each test names which slip in the oracle it would catch.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import oracle
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(seed, Bsz=2, T=9, D=3, N=4, K=4, zgate=True):
    g = np.random.default_rng(seed)
    return dict(
        x=g.normal(size=(Bsz, T, D)), z=g.normal(size=(Bsz, T, D)) if zgate else None,
        u=g.normal(size=(Bsz, T, D)), dt=g.normal(scale=0.5, size=(Bsz, T, D)),
        Bm=g.normal(size=(Bsz, T, N)), Cm=g.normal(size=(Bsz, T, N)),
        A_log=np.log(g.uniform(0.3, 6.0, size=(D, N))), D_skip=g.normal(size=D),
        dt_bias=g.normal(scale=0.3, size=D), conv_w=g.uniform(-1, 1, size=(D, K)),
        conv_b=g.normal(size=D), h0=g.normal(size=(Bsz, D, N)), s0=g.normal(size=(Bsz, D, K)))


def _scan(c, **kw):
    args = dict(u=c["u"], dt=c["dt"], A_log=c["A_log"], Bm=c["Bm"], Cm=c["Cm"], D_skip=c["D_skip"],
                z=c["z"], dt_bias=c["dt_bias"], delta_softplus=True, ssm_state=c["h0"])
    args.update(kw)
    return oracle.selective_scan_fwd(**args)


# ---------------------------------------------------------------- hand-worked fixtures

def test_golden_dyadic_scan():
    """Hand-worked example (tests/golden/scan_dyadic.json). Catches a wrong sign of A,
    a missing delta on B, a dropped D skip, a readout taken before the update."""
    f = json.load(open(os.path.join(GOLD, "scan_dyadic.json")))
    i = f["inputs"]
    A_log = np.log(np.array(i["A_log_as_log_of_multiple_of_ln2"]) * math.log(2.0))[None, :]
    y, h = oracle.selective_scan_fwd(
        u=np.array(i["u"]).reshape(1, 3, 1), dt=np.array(i["dt"]).reshape(1, 3, 1), A_log=A_log,
        Bm=np.array(i["Bm"]).reshape(1, 3, 2), Cm=np.array(i["Cm"]).reshape(1, 3, 2),
        D_skip=np.array([i["D_skip"]]), z=None, dt_bias=None, delta_softplus=False,
        ssm_state=np.array(i["h0"]).reshape(1, 1, 2))
    tol = f["tolerance_abs"]
    np.testing.assert_allclose(y.ravel(), f["expected"]["y"], rtol=0, atol=tol)
    np.testing.assert_allclose(h.ravel(), f["expected"]["h_final"], rtol=0, atol=tol)


def test_golden_conv_impulse_tap_order():
    """Impulse response fixes the tap order (tests/golden/conv_impulse.json).
    Catches reversed taps, an off-by-one window and a wrong state update."""
    f = json.load(open(os.path.join(GOLD, "conv_impulse.json")))
    w = np.array([f["w"]])
    x = np.array(f["x"]).reshape(1, 8, 1)
    u, st = oracle.conv1d_fwd(x, w, None, np.zeros((1, 1, 4)))
    c = np.array(f["expected_preactivation"])
    # silu is invertible on this range; compare u against silu of the expected pre-activation
    np.testing.assert_allclose(u.ravel(), c / (1.0 + np.exp(-c)), rtol=1e-15, atol=0)
    np.testing.assert_array_equal(st.ravel(), f["expected_state_after_T8"])
    _, st2 = oracle.conv1d_fwd(x[:, :2], w, None, np.zeros((1, 1, 4)))
    np.testing.assert_array_equal(st2.ravel(), f["expected_state_after_T2"])


# ---------------------------------------------------------------- closed forms

def test_geometric_closed_form_scan():
    """Constant delta, u, B, C: h_t = a^(t+1) h0 + dBu (1 - a^(t+1)) / (1 - a).
    Catches a wrong exponent, a missing decay of h0, a wrong D or gate."""
    T, N = 40, 5
    g = np.random.default_rng(1)
    delta, uu, zz, Dsk = 0.37, -1.3, 0.8, 0.6
    A = -g.uniform(0.2, 3.0, size=N)
    Bn, Cn, h0 = g.normal(size=N), g.normal(size=N), g.normal(size=N)
    y, h = oracle.selective_scan_fwd(
        u=np.full((1, T, 1), uu), dt=np.full((1, T, 1), delta), A_log=np.log(-A)[None, :],
        Bm=np.tile(Bn, (1, T, 1)), Cm=np.tile(Cn, (1, T, 1)), D_skip=np.array([Dsk]),
        z=np.full((1, T, 1), zz), dt_bias=None, delta_softplus=False, ssm_state=h0.reshape(1, 1, N))
    a = np.exp(delta * A)
    t1 = np.arange(1, T + 1)[:, None]
    ht = a ** t1 * h0 + delta * Bn * uu * (1 - a ** t1) / (1 - a)
    gate = zz / (1 + math.exp(-zz))
    yexp = (ht @ Cn + Dsk * uu) * gate
    np.testing.assert_allclose(y.ravel(), yexp, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(h.ravel(), ht[-1], rtol=1e-12, atol=1e-14)


def test_constant_conv_closed_form():
    """Constant input with the history pre-filled with it: u = silu(b + x * sum(w))."""
    g = np.random.default_rng(2)
    D, K, T = 5, 4, 7
    w, b = g.uniform(-1, 1, size=(D, K)), g.normal(size=D)
    xv = g.normal(size=D)
    x = np.tile(xv, (1, T, 1))
    st = np.tile(xv[:, None], (1, 1, K))
    u, _ = oracle.conv1d_fwd(x, w, b, st)
    c = b + xv * w.sum(axis=1)
    np.testing.assert_allclose(u[0], np.tile(c / (1 + np.exp(-c)), (T, 1)), rtol=1e-14)


def test_softplus_values():
    """softplus(0) = ln 2; softplus undoes the dt-bias initialisation; large/small limits."""
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-16, abs=0)
    bias, dt0 = W.dt_bias_init(4096, W.rng(0, 0, W.DT0))
    sp = np.array([oracle.softplus(float(v)) for v in W.inv_softplus(dt0)])
    np.testing.assert_allclose(sp, dt0, rtol=1e-13)
    assert oracle.softplus(50.0) == 50.0
    assert oracle.softplus(-50.0) == pytest.approx(math.exp(-50.0), rel=1e-15)
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(3.0) == pytest.approx(3.0 / (1.0 + math.exp(-3.0)), rel=1e-16)


# ---------------------------------------------------------------- brute force

def _brute_scan(c):
    """h_t = exp(A S_t) h0 + sum_{s<=t} exp(A (S_t - S_s)) delta_s B_s u_s with S_t the
    running sum of delta: the solution of the recurrence, not the recurrence."""
    Bsz, T, D = c["u"].shape
    N = c["A_log"].shape[1]
    A = -np.exp(c["A_log"])
    v = c["dt"] + c["dt_bias"]
    delta = np.logaddexp(0.0, v)
    y = np.zeros((Bsz, T, D))
    hT = np.zeros((Bsz, D, N))
    for b in range(Bsz):
        for d in range(D):
            S = np.cumsum(delta[b, :, d])
            for t in range(T):
                h = np.exp(A[d] * S[t]) * c["h0"][b, d]
                for s in range(t + 1):
                    h = h + np.exp(A[d] * (S[t] - S[s])) * delta[b, s, d] * c["Bm"][b, s] * c["u"][b, s, d]
                yv = h @ c["Cm"][b, t] + c["D_skip"][d] * c["u"][b, t, d]
                zt = c["z"][b, t, d]
                y[b, t, d] = yv * zt / (1 + np.exp(-zt))
                if t == T - 1:
                    hT[b, d] = h
    return y, hT


@pytest.mark.parametrize("seed", [3, 4])
def test_bruteforce_tiny_scan(seed):
    c = _rand_case(seed, Bsz=2, T=12, D=3, N=4)
    y, h = _scan(c)
    yb, hb = _brute_scan(c)
    np.testing.assert_allclose(y, yb, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(h, hb, rtol=1e-11, atol=1e-12)


def test_conv_toeplitz_and_numpy_convolve():
    """Conv against an explicit Toeplitz product and np.convolve on the padded window."""
    c = _rand_case(5, Bsz=2, T=10, D=3, K=4)
    u, st = oracle.conv1d_fwd(c["x"], c["conv_w"], c["conv_b"], c["s0"])
    Bsz, T, D = c["x"].shape
    K = c["conv_w"].shape[1]
    for b in range(Bsz):
        for d in range(D):
            X = np.concatenate([c["s0"][b, d], c["x"][b, :, d]])
            pre = np.convolve(X, c["conv_w"][d][::-1], mode="valid")[1:] + c["conv_b"][d]
            M = np.zeros((T, K + T))
            for t in range(T):
                M[t, t + 1:t + 1 + K] = c["conv_w"][d]
            pre2 = M @ X + c["conv_b"][d]
            np.testing.assert_allclose(pre, pre2, rtol=1e-14, atol=1e-14)
            np.testing.assert_allclose(u[b, :, d], pre / (1 + np.exp(-pre)), rtol=1e-13, atol=1e-15)
            np.testing.assert_array_equal(st[b, d], X[T:T + K])


def test_constant_delta_scan_is_iir_filter():
    """With delta constant each state is a first-order IIR filter of delta*B_t*u_t:
    checked against scipy.signal.lfilter (with the initial condition)."""
    signal = pytest.importorskip("scipy.signal")
    g = np.random.default_rng(6)
    T, N = 50, 3
    delta = 0.21
    A = -g.uniform(0.2, 2.0, size=N)
    u = g.normal(size=(1, T, 1))
    Bm, Cm, h0 = g.normal(size=(1, T, N)), g.normal(size=(1, T, N)), g.normal(size=N)
    y, h = oracle.selective_scan_fwd(u=u, dt=np.full((1, T, 1), delta), A_log=np.log(-A)[None, :],
                                     Bm=Bm, Cm=Cm, D_skip=None, z=None, dt_bias=None,
                                     delta_softplus=False, ssm_state=h0.reshape(1, 1, N))
    H = np.zeros((T, N))
    for n in range(N):
        a = math.exp(delta * A[n])
        H[:, n], _ = signal.lfilter([1.0], [1.0, -a], delta * Bm[0, :, n] * u[0, :, 0], zi=[a * h0[n]])
    np.testing.assert_allclose(y.ravel(), (H * Cm[0]).sum(axis=1), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(h.ravel(), H[-1], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- special cases

def test_zero_B_gives_skip_only():
    """B = 0 and h0 = 0: the state stays 0 and y = D u silu(z) exactly; C = 0 likewise;
    z = 0 gives y = 0 (silu(0) = 0)."""
    c = _rand_case(7)
    zero_h = np.zeros_like(c["h0"])
    expect = c["D_skip"] * c["u"] * (c["z"] / (1 + np.exp(-c["z"])))
    y, h = _scan(c, Bm=np.zeros_like(c["Bm"]), ssm_state=zero_h)
    np.testing.assert_allclose(y, expect, rtol=1e-15, atol=0)
    assert not h.any()
    y2, _ = _scan(c, Cm=np.zeros_like(c["Cm"]), ssm_state=zero_h)
    np.testing.assert_allclose(y2, expect, rtol=1e-15, atol=0)
    y3, _ = _scan(c, z=np.zeros_like(c["z"]))
    assert not y3.any()


def test_superposition_and_scaling():
    """For fixed delta, B, C and no gate, y is linear in (h0, u)."""
    c = _rand_case(8, zgate=False)
    y_h, _ = _scan(c, u=np.zeros_like(c["u"]), D_skip=c["D_skip"])
    y_u, _ = _scan(c, ssm_state=np.zeros_like(c["h0"]))
    y_both, _ = _scan(c)
    np.testing.assert_allclose(y_both, y_h + y_u, rtol=1e-12, atol=1e-13)
    y_3u, _ = _scan(c, u=3.0 * c["u"], ssm_state=np.zeros_like(c["h0"]))
    np.testing.assert_allclose(y_3u, 3.0 * y_u, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- invariants

def test_step_equals_first_scan_step():
    """The separately written step functions agree bit for bit with T=1 prefill."""
    c = _rand_case(9, T=1)
    y, h = _scan(c)
    ys, hs = oracle.ssm_step(c["u"][:, 0], c["dt"][:, 0], c["A_log"], c["Bm"][:, 0], c["Cm"][:, 0],
                             c["D_skip"], c["z"][:, 0], c["dt_bias"], c["h0"])
    np.testing.assert_array_equal(ys, y[:, 0])
    np.testing.assert_array_equal(hs, h)
    u, st = oracle.conv1d_fwd(c["x"], c["conv_w"], c["conv_b"], c["s0"])
    us, sts = oracle.conv1d_step(c["x"][:, 0], c["conv_w"], c["conv_b"], c["s0"])
    np.testing.assert_array_equal(us, u[:, 0])
    np.testing.assert_array_equal(sts, st)


def test_decode_steps_equal_prefill():
    """T decode steps from the same state reproduce a T-token prefill bit for bit."""
    c = _rand_case(10, T=11)
    y, h = _scan(c)
    u, st = oracle.conv1d_fwd(c["x"], c["conv_w"], c["conv_b"], c["s0"])
    hs, ss = c["h0"].copy(), c["s0"].copy()
    for t in range(11):
        yt, hs = oracle.ssm_step(c["u"][:, t], c["dt"][:, t], c["A_log"], c["Bm"][:, t], c["Cm"][:, t],
                                 c["D_skip"], c["z"][:, t], c["dt_bias"], hs)
        ut, ss = oracle.conv1d_step(c["x"][:, t], c["conv_w"], c["conv_b"], ss)
        np.testing.assert_array_equal(yt, y[:, t])
        np.testing.assert_array_equal(ut, u[:, t])
    np.testing.assert_array_equal(hs, h)
    np.testing.assert_array_equal(ss, st)


@pytest.mark.parametrize("cuts", [[5], [1, 2, 3], [1, 1, 1, 1, 9], [2, 13]])
def test_split_prefill_equals_full(cuts):
    """Prefill in pieces carrying both states equals one-shot prefill bit for bit,
    including pieces shorter than K-1 that exercise the conv-state shift."""
    c = _rand_case(11, T=17)
    y, h = _scan(c)
    u, st = oracle.conv1d_fwd(c["x"], c["conv_w"], c["conv_b"], c["s0"])
    edges = np.cumsum([0] + cuts + [17 - sum(cuts)])
    hs, ss = c["h0"], c["s0"]
    for a, b in zip(edges[:-1], edges[1:]):
        sl = slice(a, b)
        yp, hs = _scan(c, u=c["u"][:, sl], dt=c["dt"][:, sl], Bm=c["Bm"][:, sl], Cm=c["Cm"][:, sl],
                       z=c["z"][:, sl], ssm_state=hs)
        up, ss = oracle.conv1d_fwd(c["x"][:, sl], c["conv_w"], c["conv_b"], ss)
        np.testing.assert_array_equal(yp, y[:, sl])
        np.testing.assert_array_equal(up, u[:, sl])
    np.testing.assert_array_equal(hs, h)
    np.testing.assert_array_equal(ss, st)


def test_strided_rows_read_only_their_lane():
    """Row strides: the x lane / z lane / B,C columns read from wider rows give the same
    result as the compact tensors (in_proj and x_proj output layouts)."""
    c = _rand_case(12, D=3, N=4)
    g = np.random.default_rng(13)
    Bsz, T, D = c["u"].shape
    xz = np.concatenate([c["x"], c["z"]], axis=2)  # [B,T,2D]: x lane then z lane
    xdbl = np.concatenate([g.normal(size=(Bsz, T, 2)), c["Bm"], c["Cm"]], axis=2)
    u1, _ = oracle.conv1d_fwd(xz, c["conv_w"], c["conv_b"], c["s0"])
    u2, _ = oracle.conv1d_fwd(c["x"], c["conv_w"], c["conv_b"], c["s0"])
    np.testing.assert_array_equal(u1, u2)
    y1, _ = _scan(c, z=xz[:, :, D:], Bm=xdbl[:, :, 2:6], Cm=xdbl[:, :, 6:10])
    y2, _ = _scan(c)
    np.testing.assert_array_equal(y1, y2)


def test_channels_independent():
    """Changing one channel's inputs changes only that channel's outputs."""
    c = _rand_case(14)
    y, h = _scan(c)
    u2 = c["u"].copy()
    u2[1, :, 2] += 1.0
    y2, h2 = _scan(c, u=u2)
    diff = np.abs(y2 - y).sum(axis=1)
    assert diff[1, 2] > 0 and np.count_nonzero(diff) == 1
    assert np.count_nonzero(np.abs(h2 - h).sum(axis=2)) == 1
