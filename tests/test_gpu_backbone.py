"""The full-backbone pieces (embedding, RMSNorm, bf16 GEMMs, the layer loop) vs the f64 oracle
of oracle/backbone.py, through the C-ABI.

Bars: GEMM and RMSNorm outputs in f32 <= 1e-4 (max-abs-rel with RMS floor; the operands are
the same bf16 values on both sides, only the f32 summation order differs); a bf16 output and
the full backbone, whose activations are rounded to bf16 at every GEMM input (a value near a
rounding boundary can round either way on the two sides and propagate), <= 2e-2.
"""
import sys

import numpy as np
import pytest
import torch

import mamba_selective_scan_fwd_amd as m
import workloads as W
from oracle import backbone as ob
from oracle import oracle
from tests.parity_util import TOL_BF16, TOL_F32, dev, host, rel_err

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).cuda()


# ------------------------------------------------------------------ GEMM

GEMM_CASES = [
    # (M, N, K, a_dtype, accumulate)  -- tiles 128x128 and 64x32, ragged M/N/K, the layer shapes
    (9, 16, 32, "f32", False),
    (37, 80, 1536, "f32", False),      # x_proj shape, ragged M
    (300, 520, 100, "bf16", False),    # K not a multiple of 32, N not a multiple of 128
    (257, 3072, 768, "bf16", False),   # in_proj
    (130, 1536, 48, "f32", False),     # dt_proj: K = 48
    (200, 768, 1536, "f32", True),     # out_proj + residual
    (1, 50280, 768, "bf16", False),    # the LM head, one row
    (8, 1000, 33, "f32", False),       # few-row path, ragged K
    (3, 768, 1536, "f32", True),       # few-row path accumulating (a 1-token prefill of 3 prompts)
    (8, 200, 3000, "f32", False),      # few rows but M * K beyond the staging LDS: MFMA tiles
    (64, 3072, 768, "bf16", False),    # a decode step's in_proj (B = 64): 64 x 32 tiles
    (64, 768, 1536, "f32", True),      # a decode step's out_proj + residual
    (40, 1536, 48, "f32", False),      # dt_proj at B = 40
    (64, 50280, 768, "bf16", False),   # the head at B = 64
    (4100, 768, 1536, "bf16", True),   # out_proj + residual at a prefill's row count, ragged M
    (4096, 1000, 256, "f32", False),   # many rows, a narrow ragged N
    # plain bf16 products over many rows: ragged M and N, and K of one, two and three 32-k
    # steps (direct LDS staging only for whole 64-k slabs)
    (4100, 3000, 768, "bf16", False),
    (4096, 256, 32, "bf16", False),
    (4096, 384, 64, "bf16", False),
    (4224, 640, 96, "bf16", False),
]


@pytest.mark.parametrize("M,N,K,adt,acc", GEMM_CASES)
def test_gemm_vs_oracle(M, N, K, adt, acc):
    _say(f"case gemm M{M} N{N} K{K} A={adt} acc={acc}")
    g = np.random.default_rng(M * 7 + N + K)
    A = g.normal(size=(M, K)).astype(np.float32)
    Wt = W.bf16_round(g.normal(size=(N, K)).astype(np.float32) * 0.05)
    C0 = g.normal(size=(M, N)).astype(np.float32) if acc else np.zeros((M, N), np.float32)
    Ad = _bf16_dev(A) if adt == "bf16" else dev(A)
    C = dev(C0)
    m.mamba_gemm_bf16(Ad, _bf16_dev(Wt), C, accumulate=acc)
    torch.cuda.synchronize()
    ref = ob.gemm(A, Wt) + (C0 if acc else 0.0)
    err = rel_err(host(C), ref)
    _say(f"  err {err:.2e}")
    assert err <= TOL_F32


def test_gemm_strided_operands():
    """lda, ldw, ldc larger than the logical sizes (the layer reads the dt lane of x_proj's
    output with lda = dt_rank + 2 * d_state): untouched columns of C keep their values."""
    _say("case gemm strided")
    g = np.random.default_rng(5)
    M, N, K = 70, 96, 48
    Abig = g.normal(size=(M, 80)).astype(np.float32)
    Wbig = W.bf16_round(g.normal(size=(N, 64)).astype(np.float32))
    Cbig = np.full((M, 130), 7.0, np.float32)
    C = dev(Cbig)
    m.mamba_gemm_bf16(dev(Abig), _bf16_dev(Wbig), C, M=M, N=N, K=K, lda=80, ldw=64, ldc=130)
    torch.cuda.synchronize()
    out = host(C)
    assert rel_err(out[:, :N], ob.gemm(Abig[:, :K], Wbig[:, :K])) <= TOL_F32
    np.testing.assert_array_equal(out[:, N:], 7.0)


@pytest.mark.parametrize("M,N,K,ldw,acc", [
    (8, 520, 96, 96, True),      # 16-byte path at the row limit, last column group partly out
    (5, 300, 64, 72, False),     # 16-byte path with a strided weight row (ldw > K)
    (4, 77, 40, 44, False),      # ldw not a multiple of 8: the element-wise kernel
])
def test_gemm_few_rows_vector_and_fallback(M, N, K, ldw, acc):
    """The few-row product (M <= 8) on its 16-byte weight path and on the element-wise path,
    against the oracle; columns of C beyond N keep their values."""
    _say(f"case gemm few rows M{M} N{N} K{K} ldw{ldw} acc={acc}")
    g = np.random.default_rng(M * 31 + N + K)
    A = g.normal(size=(M, K)).astype(np.float32)
    Wbig = W.bf16_round(g.normal(size=(N, ldw)).astype(np.float32) * 0.05)
    C0 = g.normal(size=(M, N + 3)).astype(np.float32)
    C = dev(C0)
    m.mamba_gemm_bf16(dev(A), _bf16_dev(Wbig), C, M=M, N=N, K=K, ldw=ldw, ldc=N + 3, accumulate=acc)
    torch.cuda.synchronize()
    out = host(C)
    ref = ob.gemm(A, Wbig[:, :K]) + (C0[:, :N] if acc else 0.0)
    assert rel_err(out[:, :N], ref) <= TOL_F32
    np.testing.assert_array_equal(out[:, N:], C0[:, N:])


def test_gemm_empty_is_noop():
    C = torch.full((4, 4), 3.0, device="cuda")
    A = torch.zeros(0, 16, device="cuda")
    m.mamba_gemm_bf16(A, _bf16_dev(np.zeros((4, 16))), C, M=0)
    torch.cuda.synchronize()
    assert (C == 3.0).all()


# ------------------------------------------------------------------ RMSNorm, embedding

# x_proj then dt_proj of a prefill layer: (M, d_inner, dt_rank, d_state). The split-K sum
# and dt_proj run as one kernel for the first four (the 130m layer; a ragged row count; a
# narrow layer whose column split is 2; dt_rank 56, so the second 32-wide k step is part
# zero); the last three take the two-product path (dt_rank beyond 64; few rows, no split;
# d_inner not whole 64-wide slabs).
XDT_CASES = [(8192, 1536, 48, 16), (1000, 1536, 48, 16), (210, 128, 8, 16), (300, 512, 56, 16),
             (500, 640, 80, 16), (40, 1536, 48, 16), (333, 1000, 48, 16)]


@pytest.mark.parametrize("M,D,R,N", XDT_CASES)
def test_xproj_dtproj_vs_oracle(M, D, R, N):
    """xdbl against the oracle's bf16-operand product at the f32 bar. dt_proj rounds the dt
    lane of xdbl to bf16 as it enters: to make that rounding the same on both sides, each dt
    lane column of W_x has one nonzero, a power of two, so the lane is bf16(u) times a power
    of two, exact in f32 and in f64 alike (the B and C columns are dense). dt then meets the
    f32 bar against the oracle's dt_proj of its own xdbl; a wrong row, column or k index in
    either product shows as an O(1) error."""
    _say(f"case xproj_dtproj M{M} D{D} R{R} N{N}")
    xw = R + 2 * N
    g = np.random.default_rng(M + 3 * D + 7 * R)
    u = g.normal(size=(M, D)).astype(np.float32)
    Wx = W.bf16_round(g.normal(size=(xw, D)).astype(np.float32) * 0.05)
    Wx[:R] = 0.0
    cols = g.permutation(D)[:R]
    Wx[np.arange(R), cols] = np.exp2(g.integers(-3, 2, size=R)) * g.choice([-1.0, 1.0], size=R)
    Wdt = W.bf16_round(g.normal(size=(D, R)).astype(np.float32) * 0.1)
    xdbl = torch.full((M, xw), float("nan"), device="cuda")
    dt = torch.full((M, D), float("nan"), device="cuda")
    m.mamba_xproj_dtproj(dev(u), _bf16_dev(Wx), _bf16_dev(Wdt), xdbl, dt)
    torch.cuda.synchronize()
    ref_x = ob.gemm(u, Wx)
    ref_dt = ob.gemm(ref_x[:, :R], Wdt)
    ex, ed = rel_err(host(xdbl), ref_x), rel_err(host(dt), ref_dt)
    _say(f"  err xdbl {ex:.2e} dt {ed:.2e}")
    assert ex <= TOL_F32 and ed <= TOL_F32


@pytest.mark.parametrize("M,D,R,N", [(8192, 1536, 48, 16), (500, 640, 80, 16)])
def test_xproj_dtproj_delta_vs_oracle(M, D, R, N):
    """With dt_bias and softplus the call leaves the scan's delta, softplus(dt + dt_bias),
    checked against log(1 + exp(v)) in f64 (numpy's logaddexp(0, v)) of the oracle's dt plus
    the bias. The bias is the workload's dt initialisation (inverse softplus of dt in
    [1e-3, 0.1]). Covers the one-kernel path and the two-product path."""
    _say(f"case xproj_dtproj delta M{M} D{D} R{R} N{N}")
    xw = R + 2 * N
    g = np.random.default_rng(M + D + 11)
    u = g.normal(size=(M, D)).astype(np.float32)
    Wx = W.bf16_round(g.normal(size=(xw, D)).astype(np.float32) * 0.05)
    Wx[:R] = 0.0
    Wx[np.arange(R), g.permutation(D)[:R]] = np.exp2(g.integers(-3, 2, size=R)) * g.choice([-1.0, 1.0], size=R)
    Wdt = W.bf16_round(g.normal(size=(D, R)).astype(np.float32) * 0.1)
    bias, _ = W.dt_bias_init(D, g)
    bias = np.asarray(bias, np.float32)
    xdbl = torch.empty(M, xw, device="cuda")
    dt = torch.full((M, D), float("nan"), device="cuda")
    m.mamba_xproj_dtproj(dev(u), _bf16_dev(Wx), _bf16_dev(Wdt), xdbl, dt, dt_bias=dev(bias), delta_softplus=True)
    torch.cuda.synchronize()
    ref_x = ob.gemm(u, Wx)
    ref = np.logaddexp(0.0, ob.gemm(ref_x[:, :R], Wdt) + bias.astype(np.float64))
    err = rel_err(host(dt), ref)
    _say(f"  err delta {err:.2e}")
    assert err <= TOL_F32


def test_scan_takes_delta_from_xproj_dtproj():
    """The backbone hands the scan delta = softplus(dt + dt_bias) formed by the x_proj
    kernel and calls it without bias and softplus; y and the final state are the same bits
    as the scan forming delta itself from dt and the bias."""
    Bsz, T, D, R, N = 2, 300, 256, 16, 16
    xw = R + 2 * N
    g = np.random.default_rng(77)
    u = g.normal(size=(Bsz, T, D)).astype(np.float32)
    Wx = W.bf16_round(g.normal(size=(xw, D)).astype(np.float32) * 0.05)
    Wdt = W.bf16_round(g.normal(size=(D, R)).astype(np.float32) * 0.1)
    bias, _ = W.dt_bias_init(D, g)
    ud, wx, wdt, bd = dev(u), _bf16_dev(Wx), _bf16_dev(Wdt), dev(np.asarray(bias, np.float32))
    xdbl = torch.empty(Bsz * T, xw, device="cuda")
    dt = torch.empty(Bsz, T, D, device="cuda")
    delta = torch.empty(Bsz, T, D, device="cuda")
    m.mamba_xproj_dtproj(ud.view(Bsz * T, D), wx, wdt, xdbl, dt.view(Bsz * T, D))
    m.mamba_xproj_dtproj(ud.view(Bsz * T, D), wx, wdt, xdbl, delta.view(Bsz * T, D), dt_bias=bd,
                         delta_softplus=True)
    A_log = dev(np.log(np.tile(np.arange(1, N + 1, dtype=np.float32), (D, 1))))
    Dsk = dev(g.normal(size=D).astype(np.float32))
    z = dev(g.normal(size=(Bsz, T, D)).astype(np.float32))
    h0 = dev(g.normal(size=(Bsz, D, N)).astype(np.float32))
    x3 = xdbl.view(Bsz, T, xw)
    outs = []
    for dtin, b, sp in ((dt, bd, True), (delta, None, False)):
        y = torch.empty(Bsz, T, D, device="cuda")
        hs = torch.empty(Bsz, D, N, device="cuda")
        m.mamba_selective_scan_fwd(ud, dtin, b, A_log, x3[..., R:R + N], x3[..., R + N:], Dsk, z, h0, hs, y,
                                   delta_softplus=sp, workspace=m.scan_workspace(Bsz, T, D, N))
        torch.cuda.synchronize()
        outs.append((host(y), host(hs)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_xproj_dtproj_strided_u():
    """u as the x lane of a wider row (the conv output is contiguous in the backbone; the
    ABI takes any row stride that is a multiple of 8 on the fused path)."""
    M, D, R, N = 700, 1536, 48, 16
    xw = R + 2 * N
    g = np.random.default_rng(5)
    u = g.normal(size=(M, 2 * D)).astype(np.float32)
    Wx = W.bf16_round(g.normal(size=(xw, D)).astype(np.float32) * 0.05)
    Wx[:R] = 0.0
    Wx[np.arange(R), g.permutation(D)[:R]] = 0.5
    Wdt = W.bf16_round(g.normal(size=(D, R)).astype(np.float32) * 0.1)
    xdbl = torch.empty(M, xw, device="cuda")
    dt = torch.empty(M, D, device="cuda")
    ud = dev(u)
    m.mamba_xproj_dtproj(ud[:, :D], _bf16_dev(Wx), _bf16_dev(Wdt), xdbl, dt)
    torch.cuda.synchronize()
    ref_x = ob.gemm(u[:, :D], Wx)
    assert rel_err(host(xdbl), ref_x) <= TOL_F32
    assert rel_err(host(dt), ob.gemm(ref_x[:, :R], Wdt)) <= TOL_F32


# conv + x_proj + dt_proj of a prefill layer: (B, T, d_inner, d_conv, dt_rank, d_state,
# lengths). The conv runs inside x_proj's product for the first four: the 130m layer; a
# ragged T (70 = 2 x 32 + 6); 40 sequences of 2 tokens, where every workgroup holds a
# sequence start and the taps reach into the state; ragged lengths. The last two take the
# conv kernel and the split product: d_conv 3; few rows (no K split).
CXD_CASES = [(4, 2048, 1536, 4, 48, 16, None), (3, 70, 128, 4, 8, 16, None), (40, 2, 512, 4, 16, 16, None),
             (3, 70, 256, 4, 16, 16, [70, 33, 1]), (2, 300, 256, 3, 16, 16, None), (2, 5, 128, 4, 8, 16, None)]


def _cxd_inputs(Bsz, T, D, K, R, N, seed):
    g = np.random.default_rng(seed)
    xw = R + 2 * N
    x = g.normal(size=(Bsz, T, 2 * D)).astype(np.float32)   # x lane of an in_proj row: columns 0..D-1
    cw = (g.normal(size=(D, K)) * 0.5).astype(np.float32)
    cb = (g.normal(size=D) * 0.1).astype(np.float32)
    cs = g.normal(size=(Bsz, D, K)).astype(np.float32)
    Wx = W.bf16_round(g.normal(size=(xw, D)).astype(np.float32) * 0.05)
    Wdt = W.bf16_round(g.normal(size=(D, R)).astype(np.float32) * 0.1)
    return x, cw, cb, cs, Wx, Wdt


def _cxd_run(fused, x, cw, cb, cs, Wx, Wdt, lengths=None):
    Bsz, T, _ = x.shape
    D, K = cw.shape
    R = Wdt.shape[1]
    xw = Wx.shape[0]
    xd = dev(x)
    csd = dev(cs)
    u = torch.full((Bsz, T, D), float("nan"), device="cuda")
    xdbl = torch.full((Bsz * T, xw), float("nan"), device="cuda")
    dt = torch.full((Bsz * T, D), float("nan"), device="cuda")
    wx, wdt = _bf16_dev(Wx), _bf16_dev(Wdt)
    if fused:
        ln = None if lengths is None else torch.tensor(lengths, dtype=torch.int32, device="cuda")
        m.mamba_conv_xproj_dtproj(xd[..., :D], dev(cw), dev(cb), csd, u, wx, wdt, xdbl, dt, lengths=ln)
    else:
        m.mamba_conv1d_fwd(xd[..., :D], dev(cw), dev(cb), csd, u)
        m.mamba_xproj_dtproj(u.view(Bsz * T, D), wx, wdt, xdbl, dt)
    torch.cuda.synchronize()
    return host(u), host(csd), host(xdbl), host(dt)


@pytest.mark.parametrize("case", [c for c in CXD_CASES if c[6] is None],
                         ids=lambda c: "B{}T{}D{}K{}R{}".format(*c[:5]))
def test_conv_xproj_dtproj_equals_two_calls(case):
    """The one-call F4a-F4c leaves u, the conv state, xdbl and dt bit for bit as the conv
    call followed by mamba_xproj_dtproj (same tap order, same bf16 operands, same slab and
    k-step order of the MFMA sums, same in-order sum of the planes). (The conv call takes no
    per-sequence lengths: that case is checked against the oracle only.)"""
    Bsz, T, D, K, R, N, lengths = case
    _say(f"case conv_xproj_dtproj == two calls B{Bsz} T{T} D{D} K{K} R{R} N{N}")
    ins = _cxd_inputs(Bsz, T, D, K, R, N, seed=Bsz * 1000 + T + D)
    a = _cxd_run(True, *ins)
    b = _cxd_run(False, *ins)
    for name, ga, gb in zip(("u", "conv_state", "xdbl", "dt"), a, b):
        assert np.array_equal(ga, gb), f"{name} differs from the two-call path"


@pytest.mark.parametrize("case", CXD_CASES, ids=lambda c: "B{}T{}D{}K{}R{}".format(*c[:5]))
def test_conv_xproj_dtproj_vs_oracle(case):
    """u against the oracle's conv at the f32 bar, and the new conv state exactly (its
    entries are copies of x or of the old state; with lengths, the oracle's state after each
    sequence's prefix).

    xdbl and dt: u enters x_proj rounded to bf16, and where u lies next to a rounding
    midpoint the GPU's f32 u and the oracle's f64 u round to neighbouring bf16 values, one
    ulp apart (at most 2^-7 |u|). As in the x_proj test, each dt lane column of W_x has a
    single power-of-two entry, so a dt lane value is a rounded u times a power of two and
    differs from the oracle's by at most 2^-7 of itself: that is its bar. A B or C value
    moves by at most 2^-7 |u| |w| per such term; its bar allows two at the largest |u| and
    |w|, over the RMS of the reference. dt moves by at most 2^-7 |lane| |w_dt| per dt lane
    entry; its bar allows two in the same way. The bars come from the oracle's values and
    the weights only. The two-call test above pins these outputs bit for bit to calls whose
    own tests hold them to 1e-4."""
    Bsz, T, D, K, R, N, lengths = case
    _say(f"case conv_xproj_dtproj vs oracle B{Bsz} T{T} D{D} K{K} R{R} N{N} lengths={lengths}")
    x, cw, cb, cs, Wx, Wdt = _cxd_inputs(Bsz, T, D, K, R, N, seed=Bsz * 1000 + T + D + 1)
    g = np.random.default_rng(D + R)
    Wx[:R] = 0.0
    Wx[np.arange(R), g.permutation(D)[:R]] = np.exp2(g.integers(-3, 2, size=R)) * g.choice([-1.0, 1.0], size=R)
    u, st, xdbl, dt = _cxd_run(True, x, cw, cb, cs, Wx, Wdt, lengths)
    ref_u, ref_st = oracle.conv1d_fwd(x, cw, cb, cs)
    if lengths is not None:
        for bi, tb in enumerate(lengths):
            if tb < T:
                _, st_b = oracle.conv1d_fwd(x[bi:bi + 1, :tb], cw, cb, cs[bi:bi + 1])
                ref_st[bi] = st_b[0]
    assert rel_err(u, ref_u) <= TOL_F32
    assert np.array_equal(st, ref_st.astype(np.float32)), "conv state"
    ref_x = ob.gemm(ref_u.reshape(Bsz * T, D), Wx)
    ref_dt = ob.gemm(ref_x[:, :R], Wdt)
    rms = lambda a: float(np.sqrt(np.mean(np.square(a))))
    umax = float(np.abs(ref_u).max())
    tol_lane = 2.0 ** -7
    tol_bc = 2 * 2.0 ** -7 * umax * float(np.abs(Wx[R:]).max()) / rms(ref_x[:, R:])
    tol_dt = 2 * 2.0 ** -7 * float(np.abs(ref_x[:, :R]).max()) * float(np.abs(Wdt).max()) / rms(ref_dt)
    el, ebc, ed = rel_err(xdbl[:, :R], ref_x[:, :R]), rel_err(xdbl[:, R:], ref_x[:, R:]), rel_err(dt, ref_dt)
    _say(f"  err dt lane {el:.2e} (bar {tol_lane:.1e}) B|C {ebc:.2e} (bar {tol_bc:.1e}) dt {ed:.2e} "
         f"(bar {tol_dt:.1e})")
    assert el <= tol_lane and ebc <= tol_bc and ed <= tol_dt


@pytest.mark.parametrize("Dm,out", [(768, "f32"), (768, "bf16"), (100, "f32"), (2049, "f32")])
def test_rmsnorm_vs_oracle(Dm, out):
    _say(f"case rmsnorm Dm{Dm} out={out}")
    g = np.random.default_rng(Dm)
    x = (g.normal(size=(33, Dm)) * 3).astype(np.float32)
    wv = g.normal(size=Dm).astype(np.float32)
    o = torch.empty(33, Dm, device="cuda", dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    m.mamba_rmsnorm(dev(x), dev(wv), 1e-5, o)
    torch.cuda.synchronize()
    ref = ob.rmsnorm(x, wv, 1e-5)
    err = rel_err(host(o), ob.bf16(ref) if out == "bf16" else ref)
    _say(f"  err {err:.2e}")
    assert err <= (TOL_BF16 if out == "bf16" else TOL_F32)


@pytest.mark.parametrize("Dm,out", [(768, "bf16"), (768, "f32"), (1000, "f32"), (2048, "bf16")])
def test_rmsnorm_many_rows_same_bits(Dm, out):
    """A prefill's many rows take the one-wave-per-row kernel: its rows equal, bit for bit,
    the block-per-row kernel's (the same sums in the same order), and the oracle."""
    _say(f"case rmsnorm many rows Dm{Dm} out={out}")
    g = np.random.default_rng(Dm + 7)
    rows = 1100
    x = (g.normal(size=(rows, Dm)) * 2).astype(np.float32)
    wv = g.normal(size=Dm).astype(np.float32)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    xd, wd = dev(x), dev(wv)
    o_all = torch.empty(rows, Dm, device="cuda", dtype=dt)
    m.mamba_rmsnorm(xd, wd, 1e-5, o_all)           # >= 1024 rows: one wave per row
    o_few = torch.empty(40, Dm, device="cuda", dtype=dt)
    m.mamba_rmsnorm(xd[1000:1040], wd, 1e-5, o_few)  # 40 rows: one block per row
    torch.cuda.synchronize()
    assert torch.equal(o_all[1000:1040], o_few)
    ref = ob.rmsnorm(x, wv, 1e-5)
    assert rel_err(host(o_all), ob.bf16(ref) if out == "bf16" else ref) <= (TOL_BF16 if out == "bf16" else TOL_F32)


def test_rmsnorm_strided_rows():
    """The last-timestep gather: rows T * Dm apart."""
    B, T, Dm = 3, 5, 64
    x = np.random.default_rng(2).normal(size=(B, T, Dm)).astype(np.float32)
    o = torch.empty(B, Dm, device="cuda")
    xd = dev(x)
    m.mamba_rmsnorm(xd[:, T - 1], dev(np.ones(Dm)), 1e-5, o, rows=B, x_row_stride=T * Dm)
    torch.cuda.synchronize()
    assert rel_err(host(o), ob.rmsnorm(x[:, T - 1], np.ones(Dm), 1e-5)) <= TOL_F32


def test_embed_gather_exact():
    g = np.random.default_rng(3)
    E = W.bf16_round(g.normal(size=(64, 40)).astype(np.float32))
    tok = g.integers(0, 50, size=37).astype(np.int32)
    out = torch.empty(37, 40, device="cuda")
    m.mamba_embed_gather(torch.from_numpy(tok).cuda(), _bf16_dev(E), out, 50)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out), E[tok])


# ------------------------------------------------------------------ the whole backbone

def _dims(s):
    return m.BackboneDims(s.n_layers, s.d_model, s.D, s.N, s.K, s.dt_rank, s.vocab, s.vocab_padded, s.eps)


def _upload(w):
    t = {k: (_bf16_dev(v) if k in m._BACKBONE_BF16 else dev(v)) for k, v in w.items()}
    return t, m.backbone_weights_struct(t)


def _gpu_prefill(s, t, ws_struct, tokens, pieces=None, states=None):
    B, T = tokens.shape
    L, D = s.n_layers, s.D
    if states is None:
        cs = torch.zeros(L, B, D, s.K, device="cuda")
        hs = torch.zeros(L, B, D, s.N, device="cuda")
    else:
        cs, hs = (dev(a) for a in states)
    logits = torch.empty(B, s.vocab, device="cuda")
    dims = _dims(s)
    tok = torch.from_numpy(np.ascontiguousarray(tokens)).cuda()
    t0 = 0
    for n in (pieces or [T]):
        piece = tok[:, t0:t0 + n].contiguous()
        wsb = m.mamba_backbone_workspace_size(dims, B, n)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        m.mamba_backbone_prefill(dims, ws_struct, piece, cs, hs, logits, ws)
        t0 += n
    torch.cuda.synchronize()
    return host(logits), host(cs), host(hs)


def _check_backbone(what, got, ref):
    errs = [rel_err(g, r) for g, r in zip(got, ref)]
    _say(what, "logits/conv_state/ssm_state", [f"{e:.2e}" for e in errs])
    for name, e in zip(("logits", "conv_state", "ssm_state"), errs):
        assert np.isfinite(e) and e <= TOL_BF16, f"{what}: {name} error {e:.3e}"


SMALL = W.BackboneShape("small", n_layers=3, B=3, T=70, d_model=64, D=128, N=16, K=4, dt_rank=8,
                        vocab=200, vocab_padded=256)


def test_backbone_small_vs_oracle():
    _say("case backbone small L3 B3 T70 Dm64 D128")
    s = SMALL
    w = W.backbone_weights(s, seed=11)
    tok = W.backbone_tokens(s, seed=11)
    t, st = _upload(w)
    got = _gpu_prefill(s, t, st, tok)
    lg, cs, hs, _ = ob.prefill(w, tok, s.n_layers, s.D, s.N, s.dt_rank, s.vocab, s.eps)
    _check_backbone("small", got, (lg, cs, hs))


def test_backbone_small_in_pieces():
    """Prefill in three calls carrying both states equals the oracle's one-shot prefill."""
    _say("case backbone small in pieces 30+1+39")
    s = SMALL
    w = W.backbone_weights(s, seed=12)
    tok = W.backbone_tokens(s, seed=12)
    t, st = _upload(w)
    got = _gpu_prefill(s, t, st, tok, pieces=[30, 1, 39])
    lg, cs, hs, _ = ob.prefill(w, tok, s.n_layers, s.D, s.N, s.dt_rank, s.vocab, s.eps)
    _check_backbone("small pieces", got, (lg, cs, hs))


def _c4_slice(w, L):
    """The first L layers of a layer-stacked weight dict."""
    return {k: (v[:L] if v.ndim >= 2 and k not in ("embed",) else v) for k, v in w.items()}


def test_backbone_full_size_one_layer():
    """The 130m shapes (d_model 768, d_inner 1536, vocab 50280, B 4, T 2048) through one layer
    and the head: every sequence, every logit and state, at the bf16 bar."""
    s0 = W.C4
    s = W.BackboneShape("c4-1layer", n_layers=1)
    _say(f"case backbone full shapes, 1 layer, B{s.B} T{s.T}")
    w = _c4_slice(W.backbone_weights(s0), 1)
    tok = W.backbone_tokens(s0)
    t, st = _upload(w)
    got = _gpu_prefill(s, t, st, tok)
    lg, cs, hs, _ = ob.prefill(w, tok, 1, s.D, s.N, s.dt_rank, s.vocab, s.eps)
    _check_backbone("c4 1 layer", got, (lg, cs, hs))


def _normwise(g, r):
    return float(np.linalg.norm(np.asarray(g, np.float64) - r) / max(np.linalg.norm(r), 1e-30))


def _layer_slice(w, l):
    """Layer l of a layer-stacked weight dict, as a one-layer stack (embedding and norm_f kept)."""
    return {k: (v[l:l + 1] if v.ndim >= 2 and k != "embed" else v) for k, v in w.items()}


def test_backbone_full_size_per_layer():
    """Every layer of the 24-layer 130m backbone at its full shapes (B 4, T 2048), on every
    sequence, at the bf16 bar. The oracle runs the stack layer by layer in f64; the GPU runs
    layer l alone (mamba_backbone_prefill_ex over a one-layer stack, raw input rows) from the
    oracle's residual stream entering that layer, so each layer is held to 2e-2 on its own:
    its output residual stream (through norm_f, at every position), its conv and SSM states,
    and the head's logits of the last token, per sequence."""
    s0 = W.C4
    s1 = W.BackboneShape("c4-layer", n_layers=1)
    B, T = s0.B, s0.T
    _say(f"case backbone full size, per layer: L{s0.n_layers} B{B} T{T} Dm{s0.d_model}")
    w = W.backbone_weights(s0)
    tok = W.backbone_tokens(s0)
    h = np.asarray(w["embed"], np.float64)[tok]
    worst = {}
    failures = []
    for l in range(s0.n_layers):
        wl = _layer_slice(w, l)
        lg, cs, hs, h_next = ob.prefill(wl, None, 1, s0.D, s0.N, s0.dt_rank, s0.vocab, s0.eps, embeds=h)
        t, st = _upload(wl)
        g_lg, g_hid, g_cs, g_hs = _variant_run(s1, st, B, T, embeds=dev(h))
        g_lg, g_hid, g_cs, g_hs = host(g_lg), host(g_hid), host(g_cs), host(g_hs)
        ref_hid = ob.rmsnorm(h_next, w["norm_f"], s0.eps)
        errs = {}
        for b in range(B):
            for name, g_, r_ in (("hidden", g_hid[b], ref_hid[b]), ("logits", g_lg[b], lg[b]),
                                 ("conv_state", g_cs[0, b], cs[0, b]), ("ssm_state", g_hs[0, b], hs[0, b])):
                e = rel_err(g_, r_)
                errs[name] = max(errs.get(name, 0.0), e)
                if not (np.isfinite(e) and e <= TOL_BF16):
                    failures.append((l, b, name, e))
        for k, v in errs.items():
            worst[k] = max(worst.get(k, 0.0), v)
        _say(f"  layer {l:2d}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
        h = h_next
        del t, st
    _say("  worst over layers and sequences: " + " ".join(f"{k} {v:.2e}" for k, v in worst.items()))
    assert not failures, failures[:10]


def test_backbone_full_size_24_layers_drift():
    """Drift report for the 24-layer stack end to end (sequence 0; sequences are
    independent): the per-layer bar is held above, and here the layers are chained on each
    side. bf16 rounding of activations at every GEMM input turns any difference in
    summation order into different rounding decisions, which add up over depth: the oracle
    itself moves when its GEMMs sum the same bf16 products in f32 instead of f64 (about 1e-2
    normwise, 4e-2 to 2e-1 max-abs-rel). Printed: the GPU's error and that spread, max-abs-rel
    and normwise. Asserted: finite outputs and a normwise error within the bf16 bar, 2e-2."""
    s = W.C4
    _say(f"case backbone full size L{s.n_layers} T{s.T} Dm{s.d_model}, end to end, sequence 0 of {s.B}")
    w = W.backbone_weights(s)
    tok = W.backbone_tokens(s)
    t, st = _upload(w)
    got = _gpu_prefill(s, t, st, tok)
    got = (got[0][:1], got[1][:, :1], got[2][:, :1])
    ref = ob.prefill(w, tok[:1], s.n_layers, s.D, s.N, s.dt_rank, s.vocab, s.eps)[:3]
    alt = ob.prefill(w, tok[:1], s.n_layers, s.D, s.N, s.dt_rank, s.vocab, s.eps, accum="f32")[:3]
    for name, g, r, a in zip(("logits", "conv_state", "ssm_state"), got, ref, alt):
        e_max, e_nw = rel_err(g, r), _normwise(g, r)
        s_max, s_nw = rel_err(a, r), _normwise(a, r)
        _say(f"  {name}: gpu max-rel {e_max:.2e} normwise {e_nw:.2e} | oracle f32-vs-f64 "
             f"max-rel {s_max:.2e} normwise {s_nw:.2e}")
        assert np.isfinite(g).all(), name
        assert e_nw <= TOL_BF16, name


# ------------------------------------------------------------------ decode steps of the backbone

def _prefill_then_decode(s, t, st, tokens, n_prefill, graph=False):
    """GPU: prefill the first n_prefill tokens, then one decode step per remaining token
    (eager or replayed from the captured graph). Returns the logits after every step and the
    final states."""
    B, T = tokens.shape
    L = s.n_layers
    dims = _dims(s)
    cs = torch.zeros(L, B, s.D, s.K, device="cuda")
    hs = torch.zeros(L, B, s.D, s.N, device="cuda")
    logits = torch.empty(B, s.vocab, device="cuda")
    tok = torch.from_numpy(np.ascontiguousarray(tokens)).cuda()
    ws = torch.empty(m.mamba_backbone_workspace_size(dims, B, n_prefill), dtype=torch.uint8, device="cuda")
    m.mamba_backbone_prefill(dims, st, tok[:, :n_prefill].contiguous(), cs, hs, logits, ws)
    out = [host(logits)]
    wsd = torch.empty(m.mamba_backbone_decode_workspace_size(dims, B), dtype=torch.uint8, device="cuda")
    step_tok = torch.empty(B, dtype=torch.int32, device="cuda")
    g = m.DecodeGraph(dims, st, step_tok, cs, hs, logits, wsd) if graph else None
    for i in range(n_prefill, T):
        step_tok.copy_(tok[:, i])
        if graph:
            g.launch()
        else:
            m.mamba_backbone_decode_step(dims, st, step_tok, cs, hs, logits, wsd)
        out.append(host(logits))
    torch.cuda.synchronize()
    if g is not None:
        g.close()
    return out, host(cs), host(hs)


def _oracle_prefill_then_decode(s, w, tokens, n_prefill, accum="f64"):
    lg, cs, hs, _ = ob.prefill(w, tokens[:, :n_prefill], s.n_layers, s.D, s.N, s.dt_rank, s.vocab, s.eps,
                               accum=accum)
    out = [lg]
    for i in range(n_prefill, tokens.shape[1]):
        lg, cs, hs, _ = ob.prefill(w, tokens[:, i:i + 1], s.n_layers, s.D, s.N, s.dt_rank, s.vocab, s.eps,
                                   conv_state=cs, ssm_state=hs, accum=accum)
        out.append(lg)
    return out, cs, hs


@pytest.mark.parametrize("graph", [False, True])
def test_backbone_decode_small_vs_oracle(graph):
    """Prefill 20 tokens, then 6 decode steps of the 3-layer stack, eager or from the graph;
    logits after every step and the final states against the oracle (one-token prefills
    carrying the states)."""
    _say(f"case backbone decode small L3 B3, 20 + 6 tokens, graph={graph}")
    s = SMALL
    w = W.backbone_weights(s, seed=14)
    tok = W.backbone_tokens(W.BackboneShape("small26", n_layers=3, B=3, T=26, d_model=64, D=128, N=16,
                                            K=4, dt_rank=8, vocab=200, vocab_padded=256), seed=14)
    t, st = _upload(w)
    got, cs, hs = _prefill_then_decode(s, t, st, tok, 20, graph=graph)
    ref, rcs, rhs = _oracle_prefill_then_decode(s, w, tok, 20)
    for i, (g_, r_) in enumerate(zip(got, ref)):
        e = rel_err(g_, r_)
        assert e <= TOL_BF16, (i, e)
    _check_backbone("small decode", (got[-1], cs, hs), (ref[-1], rcs, rhs))


def test_backbone_decode_step_equals_one_token_prefill():
    """A decode step and a one-token prefill from the same states run the same GEMMs and the
    same conv arithmetic; only the scan's readout sum order differs (to rounding)."""
    _say("case backbone decode step == one-token prefill")
    s = SMALL
    w = W.backbone_weights(s, seed=15)
    tok = W.backbone_tokens(s, seed=15)
    t, st = _upload(w)
    dims = _dims(s)
    B, L = s.B, s.n_layers
    cs = torch.randn(L, B, s.D, s.K, device="cuda") * 0.5
    hs = torch.randn(L, B, s.D, s.N, device="cuda") * 0.5
    cs2, hs2 = cs.clone(), hs.clone()
    one = torch.from_numpy(np.ascontiguousarray(tok[:, :1])).cuda()
    lg1 = torch.empty(B, s.vocab, device="cuda")
    lg2 = torch.empty_like(lg1)
    ws = torch.empty(m.mamba_backbone_workspace_size(dims, B, 1), dtype=torch.uint8, device="cuda")
    m.mamba_backbone_prefill(dims, st, one, cs, hs, lg1, ws)
    wsd = torch.empty(m.mamba_backbone_decode_workspace_size(dims, B), dtype=torch.uint8, device="cuda")
    m.mamba_backbone_decode_step(dims, st, one[:, 0].contiguous(), cs2, hs2, lg2, wsd)
    torch.cuda.synchronize()
    assert torch.equal(cs, cs2)
    assert rel_err(host(lg2), host(lg1)) <= 1e-4
    assert rel_err(host(hs2), host(hs)) <= 1e-5


def test_backbone_decode_graph_replays_equal_eager():
    """Replays of the captured decode step, interleaved with eager steps on copies of the
    states and synchronizations, give exactly the eager results every time."""
    _say("case decode graph replays == eager steps")
    s = SMALL
    w = W.backbone_weights(s, seed=16)
    tok = W.backbone_tokens(s, seed=16)
    t, st = _upload(w)
    dims = _dims(s)
    B, L = s.B, s.n_layers
    g0 = torch.Generator(device="cuda").manual_seed(3)
    cs_g = torch.randn(L, B, s.D, s.K, device="cuda", generator=g0)
    hs_g = torch.randn(L, B, s.D, s.N, device="cuda", generator=g0)
    cs_e, hs_e = cs_g.clone(), hs_g.clone()
    lg_g = torch.empty(B, s.vocab, device="cuda")
    lg_e = torch.empty_like(lg_g)
    ws_g = torch.empty(m.mamba_backbone_decode_workspace_size(dims, B), dtype=torch.uint8, device="cuda")
    ws_e = torch.empty_like(ws_g)
    tk_g = torch.empty(B, dtype=torch.int32, device="cuda")
    tk_e = torch.empty_like(tk_g)
    graph = m.DecodeGraph(dims, st, tk_g, cs_g, hs_g, lg_g, ws_g)
    for i in range(6):
        col = torch.from_numpy(np.ascontiguousarray(tok[:, i])).cuda()
        tk_g.copy_(col)
        tk_e.copy_(col)
        graph.launch()
        m.mamba_backbone_decode_step(dims, st, tk_e, cs_e, hs_e, lg_e, ws_e)
        torch.cuda.synchronize()
        assert torch.equal(lg_g, lg_e), i
        assert torch.equal(cs_g, cs_e) and torch.equal(hs_g, hs_e), i
    graph.close()


def test_backbone_decode_full_size_per_layer():
    """One decode step of every layer of the 130m backbone at its full shapes (vocab 50280),
    B = 4, after a 24-token prefill, each layer held to the bf16 bar on its own. The oracle
    runs the prefill and the step layer by layer. The GPU step takes token ids, so layer l is
    fed the oracle's residual row entering it through the embedding: rows 0..B-1 of the
    table are replaced by those rows, rounded to bf16 (the table's type), and the tokens are
    0..B-1. The oracle evaluates the same one-layer step from the same table and the same
    states (the oracle's, after the prefill, rounded to f32 as the GPU holds them); compared
    per sequence: the new conv and SSM states and the logits (norm_f and the head over that
    table)."""
    s0 = W.C4
    B, n_pre, L = 4, 24, s0.n_layers
    s1 = W.BackboneShape("c4-decode-layer", n_layers=1, B=B, T=1)
    _say(f"case backbone decode full shapes, per layer: L{L} B{B}, {n_pre}-token prefill + 1 step")
    w = W.backbone_weights(s0)
    tok = W.backbone_tokens(s0)[:B, :n_pre + 1]
    _, cs_all, hs_all, _ = ob.prefill(w, tok[:, :n_pre], L, s0.D, s0.N, s0.dt_rank, s0.vocab, s0.eps)
    dims = _dims(s1)
    wsd = torch.empty(m.mamba_backbone_decode_workspace_size(dims, B), dtype=torch.uint8, device="cuda")
    ids = np.arange(B, dtype=np.int32)[:, None]
    step_tok = torch.from_numpy(ids[:, 0].copy()).cuda()
    h = np.asarray(w["embed"], np.float64)[tok[:, n_pre:n_pre + 1]]  # [B, 1, Dm]
    failures = []
    worst = {}
    for l in range(L):
        cs_in = cs_all[l:l + 1].astype(np.float32).astype(np.float64)
        hs_in = hs_all[l:l + 1].astype(np.float32).astype(np.float64)
        wl = _layer_slice(w, l)
        table = np.array(w["embed"], np.float32)
        table[:B] = ob.bf16(h[:, 0])
        wl["embed"] = table
        lg, cs1, hs1, _ = ob.prefill(wl, ids, 1, s0.D, s0.N, s0.dt_rank, s0.vocab, s0.eps,
                                     conv_state=cs_in, ssm_state=hs_in)
        t, st = _upload(wl)
        cs_g, hs_g = dev(cs_in), dev(hs_in)
        lg_g = torch.empty(B, s0.vocab, device="cuda")
        m.mamba_backbone_decode_step(dims, st, step_tok, cs_g, hs_g, lg_g, wsd)
        torch.cuda.synchronize()
        g_lg, g_cs, g_hs = host(lg_g), host(cs_g), host(hs_g)
        errs = {}
        for b in range(B):
            for name, g_, r_ in (("logits", g_lg[b], lg[b]), ("conv_state", g_cs[0, b], cs1[0, b]),
                                 ("ssm_state", g_hs[0, b], hs1[0, b])):
                e = rel_err(g_, r_)
                errs[name] = max(errs.get(name, 0.0), e)
                if not (np.isfinite(e) and e <= TOL_BF16):
                    failures.append((l, b, name, e))
        for k, v in errs.items():
            worst[k] = max(worst.get(k, 0.0), v)
        _say(f"  layer {l:2d}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
        # the oracle's own chain continues from its unrounded residual stream
        h = ob.prefill(_layer_slice(w, l), None, 1, s0.D, s0.N, s0.dt_rank, s0.vocab, s0.eps,
                       conv_state=cs_all[l:l + 1], ssm_state=hs_all[l:l + 1], embeds=h)[3]
        del t, st
    _say("  worst over layers and sequences: " + " ".join(f"{k} {v:.2e}" for k, v in worst.items()))
    assert not failures, failures[:10]


def test_backbone_decode_full_size_drift():
    """Drift report for the chained 24-layer decode (the per-layer bar is held above): the
    130m shapes, B = 4, a 24-token prefill and then 4 decode steps from the captured graph,
    against the oracle. Printed: the GPU's error and the oracle's own spread between f64 and
    f32 GEMM summation, max-abs-rel and normwise. Asserted: finite outputs and a normwise
    error within the bf16 bar, 2e-2."""
    s0 = W.C4
    s = W.BackboneShape("c4-decode", n_layers=24, B=4, T=28)
    _say("case backbone decode full shapes L24 B4, 24 + 4 tokens, graph, drift")
    w = W.backbone_weights(s0)
    tok = W.backbone_tokens(s0)[:, :28]
    t, st = _upload(w)
    got, cs, hs = _prefill_then_decode(s, t, st, tok, 24, graph=True)
    ref, rcs, rhs = _oracle_prefill_then_decode(s, w, tok, 24)
    alt, acs, ahs = _oracle_prefill_then_decode(s, w, tok, 24, accum="f32")
    for name, g_, r_, a_ in (("logits", got[-1], ref[-1], alt[-1]), ("conv_state", cs, rcs, acs),
                             ("ssm_state", hs, rhs, ahs)):
        e, spread = rel_err(g_, r_), rel_err(a_, r_)
        e_nw, s_nw = _normwise(g_, r_), _normwise(a_, r_)
        _say(f"  {name}: gpu max-rel {e:.2e} normwise {e_nw:.2e} | oracle f32-vs-f64 max-rel "
             f"{spread:.2e} normwise {s_nw:.2e}")
        assert np.isfinite(g_).all(), name
        assert e_nw <= TOL_BF16, name


# ------------------------------------------------------------------ prefill variants

def _variant_run(s, st, B, T, tokens=None, embeds=None, lengths=None, want_logits=True, want_hidden=True,
                 states=None):
    dims = _dims(s)
    L = s.n_layers
    if states is None:
        cs = torch.zeros(L, B, s.D, s.K, device="cuda")
        hs = torch.zeros(L, B, s.D, s.N, device="cuda")
    else:
        cs, hs = states[0].clone(), states[1].clone()
    logits = torch.empty(B, s.vocab, device="cuda") if want_logits else None
    hidden = torch.empty(B, T, s.d_model, device="cuda") if want_hidden else None
    ws = torch.empty(m.mamba_backbone_workspace_size(dims, B, T), dtype=torch.uint8, device="cuda")
    m.mamba_backbone_prefill_ex(dims, st, B, T, cs, hs, ws, tokens=tokens, embeds=embeds, lengths=lengths,
                                logits=logits, hidden=hidden)
    torch.cuda.synchronize()
    return logits, hidden, cs, hs


def test_backbone_prefill_hidden_all_positions():
    """norm_f output at every position against the oracle, and the logits equal to the plain
    prefill's."""
    _say("case backbone prefill, all-position norm_f output")
    s = SMALL
    w = W.backbone_weights(s, seed=17)
    tok = W.backbone_tokens(s, seed=17)
    t, st = _upload(w)
    tk = torch.from_numpy(tok).cuda()
    lg, hid, cs, hs = _variant_run(s, st, s.B, s.T, tokens=tk)
    lg0, cs0, hs0 = _gpu_prefill(s, t, st, tok)
    assert np.array_equal(host(lg), lg0) and np.array_equal(host(hs), hs0)
    _, _, _, h = ob.prefill(w, tok, s.n_layers, s.D, s.N, s.dt_rank, s.vocab, s.eps)
    e = rel_err(host(hid), ob.rmsnorm(h, w["norm_f"], s.eps))
    _say(f"  hidden max-rel {e:.2e}")
    assert e <= TOL_BF16


def test_backbone_prefill_from_embeds_equals_tokens():
    """The raw-input prefill started at the tokens' embedding rows is the token prefill, bit
    for bit."""
    _say("case backbone prefill from raw input rows")
    s = SMALL
    w = W.backbone_weights(s, seed=18)
    tok = W.backbone_tokens(s, seed=18)
    t, st = _upload(w)
    tk = torch.from_numpy(tok).cuda()
    emb = dev(w["embed"][tok])
    a = _variant_run(s, st, s.B, s.T, tokens=tk)
    b = _variant_run(s, st, s.B, s.T, embeds=emb)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("T,lengths", [(70, [70, 33, 1]), (400, [400, 150, 0])])
def test_backbone_ragged_batch_vs_oracle(T, lengths):
    """Right-padded sequences of different lengths in one call: each one's logits and states
    against the oracle run on that sequence alone (T = 400 runs the scan in several chunks; a
    zero length leaves that sequence's states as they were)."""
    _say(f"case backbone ragged batch T{T} lengths {lengths}")
    s = W.BackboneShape("rag", n_layers=3, B=3, T=T, d_model=64, D=128, N=16, K=4, dt_rank=8, vocab=200,
                        vocab_padded=256)
    w = W.backbone_weights(s, seed=19)
    tok = W.backbone_tokens(s, seed=19)
    t, st = _upload(w)
    g = torch.Generator(device="cuda").manual_seed(6)
    cs0 = torch.randn(3, 3, s.D, s.K, device="cuda", generator=g) * 0.5
    hs0 = torch.randn(3, 3, s.D, s.N, device="cuda", generator=g) * 0.5
    lens = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    lg, _, cs, hs = _variant_run(s, st, 3, T, tokens=torch.from_numpy(tok).cuda(), lengths=lens,
                                 want_hidden=False, states=(cs0, hs0))
    for b, n in enumerate(lengths):
        if n == 0:
            assert torch.equal(cs[:, b], cs0[:, b]) and torch.equal(hs[:, b], hs0[:, b])
            continue
        rl, rcs, rhs, _ = ob.prefill(w, tok[b:b + 1, :n], 3, s.D, s.N, s.dt_rank, s.vocab, s.eps,
                                     conv_state=host(cs0[:, b:b + 1]), ssm_state=host(hs0[:, b:b + 1]))
        errs = [rel_err(host(lg[b:b + 1]), rl), rel_err(host(cs[:, b:b + 1]), rcs), rel_err(host(hs[:, b:b + 1]), rhs)]
        _say(f"  sequence {b} (length {n}): logits/conv/ssm {[f'{e:.2e}' for e in errs]}")
        assert max(errs) <= TOL_BF16, (b, errs)


def test_backbone_decode_batch16_splitk_vs_oracle():
    """A decode batch of 16 on a wider 2-layer stack (d_model 256, d_inner 512): the
    projections run as split-K GEMMs (64 x 32 and 32 x 80 tiles, 2..8 K slices) whose partial
    planes are summed by the kernels that read them; logits and states after 4 decode steps
    against the oracle."""
    _say("case backbone decode B16, split-K projections")
    s = W.BackboneShape("wide", n_layers=2, B=16, T=12, d_model=256, D=512, N=16, K=4, dt_rank=16,
                        vocab=300, vocab_padded=320)
    w = W.backbone_weights(s, seed=20)
    tok = W.backbone_tokens(s, seed=20)
    t, st = _upload(w)
    got, cs, hs = _prefill_then_decode(s, t, st, tok, 8, graph=True)
    ref, rcs, rhs = _oracle_prefill_then_decode(s, w, tok, 8)
    for i, (g_, r_) in enumerate(zip(got, ref)):
        assert rel_err(g_, r_) <= TOL_BF16, i
    _check_backbone("decode B16", (got[-1], cs, hs), (ref[-1], rcs, rhs))


@pytest.mark.parametrize("K,N,R,B,Dm,D", [
    (3, 24, 32, 12, 128, 256),  # 8 lanes per channel (6 busy), 16-byte paths, split-K
    (2, 10, 12, 9, 128, 192),   # d_state not a multiple of 4: element-wise state and dt paths
    (4, 16, 16, 72, 128, 256),  # a batch above the split-K limit: whole products, one plane
    (4, 16, 16, 5, 128, 160),   # d_inner not a multiple of 64: conv step and x_proj as two launches
])
def test_backbone_decode_odd_shapes_vs_oracle(K, N, R, B, Dm, D):
    """Decode steps with a conv width other than 4, d_state 10 or 24 and dt_rank 12 or 32:
    the general paths of the decode kernels (window shift, lanes per channel, dt projection)
    against the oracle over 3 steps after a 5-token prefill."""
    _say(f"case backbone decode K{K} N{N} R{R} B{B}")
    s = W.BackboneShape(f"odd{K}{N}", n_layers=2, B=B, T=8, d_model=Dm, D=D, N=N, K=K, dt_rank=R,
                        vocab=150, vocab_padded=160)
    w = W.backbone_weights(s, seed=21)
    tok = W.backbone_tokens(s, seed=21)
    t, st = _upload(w)
    got, cs, hs = _prefill_then_decode(s, t, st, tok, 5)
    ref, rcs, rhs = _oracle_prefill_then_decode(s, w, tok, 5)
    for i, (g_, r_) in enumerate(zip(got, ref)):
        assert rel_err(g_, r_) <= TOL_BF16, i
    _check_backbone(f"decode K{K} N{N}", (got[-1], cs, hs), (ref[-1], rcs, rhs))
