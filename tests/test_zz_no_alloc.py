"""mamba_conv_scan_fwd_noalloc, the conv + scan prefill that allocates nothing (its chunk
summaries go to the library's fixed device scratch), through the C-ABI: its outputs equal
those of mamba_conv_scan_fwd with a caller-owned workspace bit for bit (the same kernels run
on the same inputs), on calls in a row, each after the first on a smaller input. After the
first call on the device, which sets the scratch up, the calls leave the device's free memory
unchanged."""
import sys

import numpy as np
import pytest
import torch

import mamba_selective_scan_fwd_amd as m
import workloads as W
from tests.parity_util import dev

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _inputs(shape, io, seed):
    inp = W.prefill_inputs(shape, seed=seed, random_state=True)
    t = {k: dev(inp[k], io) for k in ("x", "z", "dt", "Bm", "Cm")}
    t.update({k: dev(inp[k]) for k in ("conv_w", "conv_b", "dt_bias", "A_log", "D_skip",
                                        "conv_state", "ssm_state")})
    return t


def _buffers(t, io):
    B, T, D = t["x"].shape
    iod = torch.bfloat16 if io == "bf16" else torch.float32
    return dict(u=torch.empty(B, T, D, dtype=iod, device="cuda"),
                y=torch.empty(B, T, D, dtype=iod, device="cuda"),
                conv_state=t["conv_state"].clone(), ssm_state=t["ssm_state"].clone())


def _run(t, o, workspace=None):
    """One conv + scan call into the buffers o (states carried in place); no workspace: the
    no-allocation entry point."""
    args = (t["x"], t["conv_w"], t["conv_b"], o["conv_state"], t["dt"], t["dt_bias"], t["A_log"],
            t["Bm"], t["Cm"], t["D_skip"], t["z"], o["ssm_state"], o["ssm_state"], o["y"])
    if workspace is None:
        m.mamba_conv_scan_fwd_noalloc(*args, u=o["u"])
    else:
        m.mamba_conv_scan_fwd(*args, u=o["u"], workspace=workspace)
    return o


# the 130m-shaped layer (23 chunks, 2.4 MB of scratch), then smaller inputs that still span
# several chunks and a ragged channel tail
SHAPES = [
    (W.C1, "f32", 0),
    (W.PrefillShape("c-small", B=2, T=700, D=320), "f32", 1),
    (W.PrefillShape("c-small-bf16", B=3, T=515, D=200, io="bf16"), "bf16", 2),
]


def test_noalloc_equals_workspace_call_twice_in_a_row():
    cases = [(s, io, _inputs(s, io, seed)) for s, io, seed in SHAPES]
    refs = []
    for s, io, t in cases:
        B, T, D = t["x"].shape
        refs.append(_run(t, _buffers(t, io), workspace=m.scan_workspace(B, T, D, t["A_log"].shape[1])))
    # every output buffer exists before the no-allocation calls
    first = _buffers(cases[0][2], cases[0][1])
    outs = [_buffers(t, io) for _, io, t in cases]
    torch.cuda.synchronize()
    # the first call on the device sets the scratch up: the runtime loads the library's
    # scratch module there (the 16 MiB array), once per process and device
    free_a = torch.cuda.mem_get_info()[0]
    _run(cases[0][2], first)
    torch.cuda.synchronize()
    _say(f"case noalloc set-up call: device free memory {free_a} -> {torch.cuda.mem_get_info()[0]}")
    # (torch.equal allocates temporaries through torch's caching allocator, so every
    # comparison runs before the free memory is taken or after it is taken again)
    for k in ("u", "y", "conv_state", "ssm_state"):
        assert torch.equal(first[k], refs[0][k]), ("set-up call", k)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    # after it, calls allocate nothing: the largest case, then two smaller ones
    for (s, io, t), o in zip(cases, outs):
        B, T, D = t["x"].shape
        need = m.load_library().mamba_selective_scan_workspace_size(B, T, D, t["A_log"].shape[1])
        _say(f"case noalloc {s.name} B{B} T{T} D{D} io={io}, scan workspace {need} bytes")
        assert need > 0, "the case should span several chunks"
        _run(t, o)
        torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    for (s, io, _), ref, out in zip(cases, refs, outs):
        for k in ("u", "y", "conv_state", "ssm_state"):
            assert torch.equal(out[k], ref[k]), (s.name, k)
    _say(f"  device free memory before/after the calls: {free0} / {free1}")
    assert free1 == free0, f"device free memory moved by {free0 - free1} bytes"
