"""Pins of the backbone oracle (oracle/backbone.py): closed forms and invariants that do not
come from the oracle itself."""
import math

import numpy as np
import pytest
import torch

from oracle import backbone as ob
from oracle import oracle
import workloads as W


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    v = np.concatenate([g.normal(size=5000) * 10.0 ** g.integers(-30, 30, size=5000),
                        [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 3.4e38]])
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ob.bf16(v), ref)


def test_rmsnorm_constant_row_closed_form():
    c, eps = 0.37, 1e-5
    out = ob.rmsnorm(np.full((3, 16), c), np.ones(16), eps)
    np.testing.assert_allclose(out, c / math.sqrt(c * c + eps), rtol=1e-15)
    w = np.arange(1, 17, dtype=np.float64)
    np.testing.assert_allclose(ob.rmsnorm(np.full(16, c), w, eps), w * c / math.sqrt(c * c + eps), rtol=1e-15)


def test_gemm_is_bf16_product_brute_force():
    g = np.random.default_rng(1)
    A, Wm = g.normal(size=(5, 7)), g.normal(size=(3, 7))
    out = ob.gemm(A, Wm)
    a, w = ob.bf16(A), ob.bf16(Wm)
    ref = np.array([[sum(a[i, k] * w[j, k] for k in range(7)) for j in range(3)] for i in range(5)])
    np.testing.assert_allclose(out, ref, rtol=1e-14, atol=1e-15)


def _tiny(L=2):
    s = W.BackboneShape("t", n_layers=L, B=2, T=9, d_model=16, D=32, N=4, K=4, dt_rank=3, vocab=40,
                        vocab_padded=64)
    return s, W.backbone_weights(s, seed=3), W.backbone_tokens(s, seed=3)


def test_zero_out_proj_keeps_residual_stream():
    """With out_proj = 0 every layer adds nothing: the hidden state stays the embedding and
    the logits are the head applied to norm_f of the last token's embedding."""
    s, w, tok = _tiny()
    w["out_proj"][:] = 0.0
    logits, _, _, h = ob.prefill(w, tok, s.n_layers, s.D, s.N, s.dt_rank, s.vocab, s.eps)
    np.testing.assert_array_equal(h, w["embed"].astype(np.float64)[tok])
    last = w["embed"].astype(np.float64)[tok[:, -1]]
    nl = last / np.sqrt(np.mean(last * last, axis=1, keepdims=True) + s.eps)
    np.testing.assert_allclose(logits, ob.bf16(nl) @ w["embed"][:s.vocab].astype(np.float64).T, rtol=1e-12)


def test_layer_is_the_single_layer_chain():
    """One layer of the backbone equals the hand-chained pieces: rmsnorm -> in_proj -> conv ->
    x_proj -> dt_proj -> scan -> out_proj -> residual."""
    s, w, tok = _tiny(L=1)
    logits, cs, hs, h = ob.prefill(w, tok, 1, s.D, s.N, s.dt_rank, s.vocab, s.eps)
    e = w["embed"].astype(np.float64)[tok]
    xn = ob.bf16(ob.rmsnorm(e, w["norm_w"][0], s.eps))
    proj = xn @ w["in_proj"][0].astype(np.float64).T
    u, _ = oracle.conv1d_fwd(proj[..., :s.D], w["conv_w"][0], w["conv_b"][0], np.zeros((2, s.D, 4)))
    xdbl = ob.bf16(u) @ w["x_proj"][0].astype(np.float64).T
    dt = ob.bf16(xdbl[..., :s.dt_rank]) @ w["dt_proj"][0].astype(np.float64).T
    y, _ = oracle.selective_scan_fwd(u, dt, w["A_log"][0], xdbl[..., 3:7], xdbl[..., 7:11], w["D_skip"][0],
                                     proj[..., s.D:], w["dt_bias"][0], True, None)
    np.testing.assert_allclose(h, e + ob.bf16(y) @ w["out_proj"][0].astype(np.float64).T, rtol=1e-12, atol=1e-15)


def test_prefill_in_two_pieces_equals_one():
    """Prefill carries both states per layer: two prompts pieces equal one prompt."""
    s, w, tok = _tiny()
    full, cs, hs, _ = ob.prefill(w, tok, s.n_layers, s.D, s.N, s.dt_rank, s.vocab, s.eps)
    _, cs1, hs1, _ = ob.prefill(w, tok[:, :4], s.n_layers, s.D, s.N, s.dt_rank, s.vocab, s.eps)
    two, cs2, hs2, _ = ob.prefill(w, tok[:, 4:], s.n_layers, s.D, s.N, s.dt_rank, s.vocab, s.eps,
                                  conv_state=cs1, ssm_state=hs1)
    np.testing.assert_array_equal(two, full)
    np.testing.assert_array_equal(cs2, cs)
    np.testing.assert_array_equal(hs2, hs)


def test_backbone_weight_recipe():
    s = W.BackboneShape("t", n_layers=2, B=2, T=9, d_model=16, D=32, N=4, K=4, dt_rank=3, vocab=40, vocab_padded=64)
    w = W.backbone_weights(s)
    assert w["embed"].shape == (64, 16) and not w["embed"][40:].any()
    for k in ("embed", "in_proj", "x_proj", "dt_proj", "out_proj"):
        np.testing.assert_array_equal(W.bf16_round(w[k]), w[k])
    assert w["in_proj"].shape == (2, 64, 16) and w["x_proj"].shape == (2, 11, 32)
    assert abs(w["in_proj"].std() - 0.02) < 0.004
    tok = W.backbone_tokens(s)
    assert tok.dtype == np.int32 and tok.min() >= 0 and tok.max() < 40


def test_gemm_f32_accumulation_is_close():
    """The f32-summed evaluation differs from the f64 definition only by summation rounding."""
    g = np.random.default_rng(4)
    A, Wm = g.normal(size=(20, 700)), g.normal(size=(30, 700))
    a = ob.gemm(A, Wm, "f32")
    r = ob.gemm(A, Wm)
    assert np.max(np.abs(a - r)) <= 1e-5 * np.sqrt(700) * np.max(np.abs(r)) and not np.array_equal(a, r)


def test_prefill_from_embedding_rows_equals_token_prefill():
    """The raw-input prefill started at the embedding rows of the tokens is the token prefill."""
    s, w, tok = _tiny()
    a = ob.prefill(w, tok, s.n_layers, s.D, s.N, s.dt_rank, s.vocab, s.eps)
    b = ob.prefill(w, None, s.n_layers, s.D, s.N, s.dt_rank, s.vocab, s.eps,
                   embeds=w["embed"].astype(np.float64)[tok])
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
