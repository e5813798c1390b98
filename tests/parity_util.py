"""Helpers shared by the GPU parity tests: device upload, the error metric, and running one
prefill layer through the HIP library and through the oracle on the same seeded inputs.

The oracle always starts from the generated inputs (x, dt, z, B, C, parameters, states):
it never sees an intermediate produced on the GPU.
"""
from __future__ import annotations

import numpy as np
import torch

import mamba_selective_scan_fwd_amd as m
from oracle import oracle

# Bars: max-abs-rel error with an RMS floor (see rel_err).
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def rel_err(g, r) -> float:
    """max_i |g_i - r_i| / max(|r_i|, rms(r)): relative per element, with the RMS of the
    reference as a floor so that entries near zero cannot inflate it."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    floor = max(float(np.sqrt(np.mean(r * r))), 1e-30)
    return float(np.max(np.abs(g - r) / np.maximum(np.abs(r), floor)))


def tol(io: str) -> float:
    return TOL_BF16 if io == "bf16" else TOL_F32


def dev(a, io: str = "f32", device="cuda"):
    """Upload an f32 numpy array; as bf16 when io == 'bf16' (values are already bf16-exact)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if io == "bf16":
        t = t.to(torch.bfloat16)
    return t.to(device)


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def gpu_layer(inp: dict, io: str, chunks=None, in_place_state=True, stream=None, fused=False):
    """conv1d_fwd then selective_scan_fwd on the GPU (fused: one mamba_conv_scan_fwd call,
    u written too). chunks: list of T-piece lengths to run the prefill in several calls
    carrying both states (None: one call).
    Returns dict of torch tensors: u, y, conv_state, ssm_state."""
    B, T, D = inp["x"].shape
    N = inp["A_log"].shape[1]
    iod = torch.bfloat16 if io == "bf16" else torch.float32
    x, z, dt = dev(inp["x"], io), dev(inp["z"], io), dev(inp["dt"], io)
    Bm, Cm = dev(inp["Bm"], io), dev(inp["Cm"], io)
    p = {k: dev(inp[k]) for k in ("conv_w", "conv_b", "dt_bias", "A_log", "D_skip")}
    conv_state = dev(inp["conv_state"])
    ssm_state = dev(inp["ssm_state"])
    u = torch.empty(B, T, D, dtype=iod, device="cuda")
    y = torch.empty(B, T, D, dtype=iod, device="cuda")
    pieces = [T] if chunks is None else list(chunks)
    assert sum(pieces) == T
    t0 = 0
    for n in pieces:
        sl = slice(t0, t0 + n)
        # one [B, n, .] buffer per piece, as a caller prefilling a prompt piece by piece holds
        if n == T:
            xs, zs, dts, Bs, Cs = x, z, dt, Bm, Cm
        else:
            xs, zs, dts = x[:, sl].contiguous(), z[:, sl].contiguous(), dt[:, sl].contiguous()
            Bs, Cs = Bm[:, sl].contiguous(), Cm[:, sl].contiguous()
        us = torch.empty(B, n, D, dtype=iod, device="cuda")
        ys = torch.empty(B, n, D, dtype=iod, device="cuda")
        ws = m.scan_workspace(B, n, D, N)
        out_state = ssm_state if in_place_state else torch.empty_like(ssm_state)
        if fused:
            m.mamba_conv_scan_fwd(xs, p["conv_w"], p["conv_b"], conv_state, dts, p["dt_bias"],
                                  p["A_log"], Bs, Cs, p["D_skip"], zs, ssm_state, out_state, ys,
                                  u=us, workspace=ws, stream=stream)
        else:
            m.mamba_conv1d_fwd(xs, p["conv_w"], p["conv_b"], conv_state, us, stream=stream)
            m.mamba_selective_scan_fwd(us, dts, p["dt_bias"], p["A_log"], Bs, Cs, p["D_skip"], zs,
                                       ssm_state, out_state, ys, workspace=ws, stream=stream)
        ssm_state = out_state
        u[:, sl] = us
        y[:, sl] = ys
        t0 += n
    torch.cuda.synchronize()
    return dict(u=u, y=y, conv_state=conv_state, ssm_state=ssm_state)


def oracle_layer(inp: dict, channels=None):
    """The oracle's conv + scan on the generated inputs. channels: None for all, or a list of
    (b, d) pairs; then each returned array holds only those channels:
    u, y: [n_ch, T]; conv_state: [n_ch, K]; ssm_state: [n_ch, N]."""
    if channels is None:
        u, cs = oracle.conv1d_fwd(inp["x"], inp["conv_w"], inp["conv_b"], inp["conv_state"])
        y, hs = oracle.selective_scan_fwd(u, inp["dt"], inp["A_log"], inp["Bm"], inp["Cm"],
                                          inp["D_skip"], inp["z"], inp["dt_bias"], True,
                                          inp["ssm_state"])
        return dict(u=u, y=y, conv_state=cs, ssm_state=hs)
    out = {k: [] for k in ("u", "y", "conv_state", "ssm_state")}
    for b, d in channels:
        sel = slice(d, d + 1)
        u, cs = oracle.conv1d_fwd(inp["x"][b:b + 1, :, sel], inp["conv_w"][sel], inp["conv_b"][sel],
                                  inp["conv_state"][b:b + 1, sel])
        y, hs = oracle.selective_scan_fwd(u, inp["dt"][b:b + 1, :, sel], inp["A_log"][sel],
                                          inp["Bm"][b:b + 1], inp["Cm"][b:b + 1], inp["D_skip"][sel],
                                          inp["z"][b:b + 1, :, sel], inp["dt_bias"][sel], True,
                                          inp["ssm_state"][b:b + 1, sel])
        out["u"].append(u[0, :, 0])
        out["y"].append(y[0, :, 0])
        out["conv_state"].append(cs[0, 0])
        out["ssm_state"].append(hs[0, 0])
    return {k: np.stack(v) for k, v in out.items()}


def pick_channels(B: int, D: int, n: int, seed: int = 0):
    """A seeded sample of (b, d) channels that always includes the corners."""
    g = np.random.default_rng(seed)
    fixed = {(0, 0), (0, D - 1), (B - 1, 0), (B - 1, D - 1), (B // 2, D // 2)}
    while len(fixed) < n:
        fixed.add((int(g.integers(B)), int(g.integers(D))))
    return sorted(fixed)


def gather_channels(gpu: dict, channels):
    """GPU results at the sampled channels, in the layout oracle_layer returns."""
    bs = torch.tensor([c[0] for c in channels])
    ds = torch.tensor([c[1] for c in channels])
    return dict(
        u=host(gpu["u"][bs, :, ds]), y=host(gpu["y"][bs, :, ds]),
        conv_state=host(gpu["conv_state"][bs, ds]), ssm_state=host(gpu["ssm_state"][bs, ds]))
