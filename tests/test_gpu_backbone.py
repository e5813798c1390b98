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


def test_gemm_empty_is_noop():
    C = torch.full((4, 4), 3.0, device="cuda")
    A = torch.zeros(0, 16, device="cuda")
    m.mamba_gemm_bf16(A, _bf16_dev(np.zeros((4, 16))), C, M=0)
    torch.cuda.synchronize()
    assert (C == 3.0).all()


# ------------------------------------------------------------------ RMSNorm, embedding

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


def test_backbone_full_size_24_layers():
    """The whole 24-layer backbone on sequence 0 of the batch-4 workload (sequences are
    independent). Across 24 layers the bf16 rounding of activations at every GEMM input turns
    any difference in summation order into different rounding decisions, which then add up
    layer after layer: the oracle itself moves by several 1e-2 when its GEMMs sum the same
    bf16 products in f32 instead of f64. The bar is three times that spread, measured here
    between the two oracle evaluations, per output and per metric (max-abs-rel and normwise);
    the 2e-2 bar itself is met at one layer (test above) and on the three-layer stack."""
    s = W.C4
    _say(f"case backbone full size L{s.n_layers} T{s.T} Dm{s.d_model}, batch element 0 of {s.B}")
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
        assert np.isfinite(e_max) and e_max <= max(TOL_BF16, 3 * s_max), name
        assert e_nw <= max(TOL_BF16, 3 * s_nw), name
