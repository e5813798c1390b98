"""Mamba-3 SISO decode step on the GPU (mamba3_siso_step through the C-ABI) against the f64
oracle (oracle/mamba3.py), element by element on the same seeded inputs: the gated output
and all four carried states, over several consecutive steps, for shapes that exercise every
lane layout (d_state 4 .. 256), ragged headdim, several groups, partial and no RoPE, the
plain silu gate, strided rows, and the full 24-layer B=64 workload on sampled (layer,
sequence) pairs. Bar: 1e-4 max-abs-rel with the RMS floor (f32 I/O)."""
import numpy as np
import pytest

import workloads as W
from oracle import mamba3 as o3
from parity_util import rel_err

pytestmark = pytest.mark.gpu
TOL = 1e-4

CASES = [
    # name, L, B, nheads, headdim, d_state, ngroups, n_angles, gate_norm
    ("lpr4_groups", 2, 3, 4, 16, 16, 2, 8, True),
    ("head64_ds128", 1, 2, 2, 64, 128, 1, 64, True),
    ("ds48_hd24_partial_rope_silu", 2, 2, 3, 24, 48, 1, 5, False),
    ("max_ds256_hd256_no_rope", 1, 1, 2, 256, 256, 2, 0, True),
    ("min_ds4_group_per_head", 2, 2, 4, 8, 4, 4, 2, False),
    ("ds8_hd33", 1, 3, 2, 33, 8, 1, 4, True),
]


def oracle_params(p):
    q = {k: v for k, v in p.items() if k != "gate_norm_w"}
    q["gate_w"] = p["gate_norm_w"]
    return q


def run_steps(shape, steps, pad=0):
    import torch
    import mamba_selective_scan_fwd_amd as m

    p = W.m3_params(shape, seed=3)
    st = W.m3_states(shape, seed=3, random=True)
    dev = {k: (None if v is None else torch.from_numpy(v).cuda()) for k, v in p.items()}
    gst = {k: torch.from_numpy(v).cuda() for k, v in st.items()}
    ost = {k: v.astype(np.float64) for k, v in st.items()}
    kw = dict(nheads=shape.nheads, headdim=shape.headdim, d_state=shape.d_state,
              ngroups=shape.ngroups, n_angles=shape.na, a_floor=shape.a_floor)
    for step in range(steps):
        proj = W.m3_proj(shape, step=step, seed=3)
        buf = torch.zeros((shape.L, shape.B, shape.width + pad), dtype=torch.float32, device="cuda")
        buf[..., :shape.width] = torch.from_numpy(proj).cuda()
        out = torch.full((shape.L, shape.B, shape.d_inner), float("nan"), device="cuda")
        m.mamba3_siso_step(buf[..., :shape.width], dev, shape.a_floor, gst["ssm"], gst["k"], gst["v"],
                           gst["angle"], out, shape.ngroups, shape.na)
        torch.cuda.synchronize()
        ref = o3.siso_step(proj, oracle_params(p), ost["ssm"], ost["k"], ost["v"], ost["angle"], **kw)
        ost = dict(zip(("ssm", "k", "v", "angle"), ref[1:]))
        yield step, out.cpu().numpy(), {k: v.cpu().numpy() for k, v in gst.items()}, ref[0], ost


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_m3_step_vs_oracle(case):
    name, L, B, nh, hd, ds, ng, na, gate = case
    shape = W.Mamba3Shape(name, L=L, B=B, nheads=nh, headdim=hd, d_state=ds, ngroups=ng,
                          n_angles=na, gate_norm=gate)
    for step, out, gst, ref_out, ost in run_steps(shape, 3):
        print(f"{name} step {step}", flush=True)
        assert not np.isnan(out).any()
        assert rel_err(out, ref_out) < TOL, (step, rel_err(out, ref_out))
        for k in ("ssm", "k", "v", "angle"):
            assert rel_err(gst[k], ost[k]) < TOL, (step, k, rel_err(gst[k], ost[k]))


def test_m3_step_strided_rows():
    shape = W.Mamba3Shape("strided", L=2, B=2, nheads=2, headdim=16, d_state=32, n_angles=8)
    for step, out, gst, ref_out, ost in run_steps(shape, 2, pad=7):
        assert rel_err(out, ref_out) < TOL
        assert rel_err(gst["ssm"], ost["ssm"]) < TOL


def test_m3_step_empty_is_noop():
    import torch
    import mamba_selective_scan_fwd_amd as m

    shape = W.Mamba3Shape("empty", L=0, B=4, nheads=2, headdim=8, d_state=16)
    p = {k: (None if v is None else torch.zeros(1, device="cuda")) for k, v in W.m3_params(
        W.Mamba3Shape("p", L=1, B=1, nheads=2, headdim=8, d_state=16)).items()}
    z = lambda *s: torch.zeros(s, device="cuda")
    m.mamba3_siso_step(z(0, 4, shape.width), p, 1e-4, z(0, 4, 2, 8, 16), z(0, 4, 2, 16), z(0, 4, 2, 8),
                       z(0, 4, 2, 8), z(0, 4, 16), 1, 8)
    torch.cuda.synchronize()


def test_m3_step_full_size_sampled():
    """The 24-layer, B = 64 workload (24 heads x 64 x 128 states per sequence) in the launch
    configuration the benchmark times, two steps from random states, checked on sampled
    (layer, sequence) pairs (every other pair is still computed)."""
    import torch
    import mamba_selective_scan_fwd_amd as m

    shape = W.C5
    L, B = shape.L, shape.B
    p = W.m3_params(shape, seed=5)
    dev = {k: (None if v is None else torch.from_numpy(v).cuda()) for k, v in p.items()}
    g = W.torch_generator(5, 5, W.M3_STATE)
    gst = dict(ssm=torch.randn((L, B, shape.nheads, shape.headdim, shape.d_state), generator=g, device="cuda"),
               k=torch.randn((L, B, shape.nheads, shape.d_state), generator=g, device="cuda"),
               v=torch.randn((L, B, shape.nheads, shape.headdim), generator=g, device="cuda"),
               angle=torch.rand((L, B, shape.nheads, shape.na), generator=g, device="cuda") * 6.0 - 3.0)
    pairs = [(0, 0), (L - 1, B - 1), (7, 33), (13, 5), (20, 62)]
    ost = {k: np.stack([v[l, b].cpu().numpy() for l, b in pairs])[:, None, None].astype(np.float64)
           for k, v in gst.items()}
    kw = dict(nheads=shape.nheads, headdim=shape.headdim, d_state=shape.d_state,
              ngroups=shape.ngroups, n_angles=shape.na, a_floor=shape.a_floor)
    out = torch.empty((L, B, shape.d_inner), device="cuda")
    for step in range(2):
        print(f"c5 step {step}", flush=True)
        proj = torch.from_numpy(W.m3_proj(shape, step=step, seed=5)).cuda()
        m.mamba3_siso_step(proj, dev, shape.a_floor, gst["ssm"], gst["k"], gst["v"], gst["angle"], out,
                           shape.ngroups, shape.na)
        torch.cuda.synchronize()
        for i, (l, b) in enumerate(pairs):
            lp = {k: (None if v is None else v[l:l + 1]) for k, v in oracle_params(p).items()}
            ref = o3.siso_step(proj[l, b].cpu().numpy()[None, None], lp, ost["ssm"][i], ost["k"][i],
                               ost["v"][i], ost["angle"][i], **kw)
            for k, r in zip(("ssm", "k", "v", "angle"), ref[1:]):
                ost[k][i] = r
            assert rel_err(out[l, b].cpu().numpy(), ref[0][0, 0]) < TOL, (step, l, b)
            for k in ("ssm", "k", "v", "angle"):
                assert rel_err(gst[k][l, b].cpu().numpy(), ost[k][i][0, 0]) < TOL, (step, l, b, k)
