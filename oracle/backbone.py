"""f64 oracle of the full Mamba-1 backbone prefill (embedding, 24 layers, norm_f, tied head).

TEST INFRASTRUCTURE, like the rest of oracle/: only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may use it.

The layer follows the prefill chain of the pages (prefill.rs page of mamba-rs 0.6.4,
prefill_body: RMSNorm, in_proj, conv over the x lane, x_proj, dt_proj with its bias applied as
the scan's dt_bias, the scan gated by the z lane, out_proj, residual add; then norm_f on the
last timestep and the tied head of gpu_lm.rs, mamba-rs 0.7.1). Everything is f64; the only
rounding emulated is bf16 at the GEMM operands (weights are bf16; activations are rounded as
they enter a GEMM), which is the stated precision of the backbone. Conv and scan come from the
C oracle (oracle.py).
"""
from __future__ import annotations

import numpy as np

from oracle import oracle


def bf16(x) -> np.ndarray:
    """Round to the nearest bf16 (ties to even), through f32, returned as f64."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    b = f.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32).astype(np.float64)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = np.nan
    return out


def rmsnorm(x, w, eps) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w over the last axis."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, np.float64)


def gemm(A, W, accum: str = "f64") -> np.ndarray:
    """A @ W^T with both operands rounded to bf16 (W in nn.Linear layout [out, in]).
    accum 'f64' is the definition; 'f32' sums the same bf16 products in f32, a second correct
    evaluation order used only to measure how far rounding-order differences carry through a
    deep stack."""
    if accum == "f32":
        return (bf16(A).astype(np.float32) @ bf16(W).T.astype(np.float32)).astype(np.float64)
    return bf16(A) @ bf16(W).T


def prefill(w: dict, tokens, n_layers: int, d_inner: int, d_state: int,
            dt_rank: int, vocab: int, eps: float, conv_state=None, ssm_state=None,
            accum: str = "f64", embeds=None):
    """Returns (logits [B, vocab], conv_state [L,B,D,K], ssm_state [L,B,D,N], hidden [B,T,Dm]),
    hidden being the residual stream before norm_f. embeds: [B, T, Dm] raw input rows used in
    place of the embedding of `tokens` (the raw-input prefill). accum: the GEMMs' summation
    precision (see gemm)."""
    def gemm_(A, W):
        return gemm(A, W, accum)

    if embeds is not None:
        h = np.array(embeds, np.float64)  # [B, T, Dm]
    else:
        h = np.asarray(w["embed"], np.float64)[tokens]
    Bsz, T = h.shape[:2]
    D, N, R = d_inner, d_state, dt_rank
    K = w["conv_w"].shape[2]
    cs_all = np.zeros((n_layers, Bsz, D, K)) if conv_state is None else np.array(conv_state, np.float64)
    hs_all = np.zeros((n_layers, Bsz, D, N)) if ssm_state is None else np.array(ssm_state, np.float64)
    for l in range(n_layers):
        xn = rmsnorm(h, w["norm_w"][l], eps)
        proj = gemm_(xn, w["in_proj"][l])  # [B, T, 2D]: x lane | z lane
        u, cs = oracle.conv1d_fwd(proj[..., :D], w["conv_w"][l], w["conv_b"][l], cs_all[l])
        xdbl = gemm_(u, w["x_proj"][l])  # [B, T, R + 2N]: dt lane | B | C
        dt = gemm_(xdbl[..., :R], w["dt_proj"][l])
        y, hs = oracle.selective_scan_fwd(u, dt, w["A_log"][l], xdbl[..., R:R + N], xdbl[..., R + N:],
                                          w["D_skip"][l], proj[..., D:], w["dt_bias"][l], True,
                                          hs_all[l])
        h = h + gemm_(y, w["out_proj"][l])
        cs_all[l], hs_all[l] = cs, hs
    last = rmsnorm(h[:, T - 1], w["norm_f"], eps)
    logits = gemm_(last, np.asarray(w["embed"])[:vocab])
    return logits, cs_all, hs_all, h
