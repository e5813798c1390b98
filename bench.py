#!/usr/bin/env python3
"""Throughput of the Mamba-1 selective-scan hot path on one MI355X.

A step is one pass of the prefill hot path over one batch of synthetic input already
resident in HBM: mamba_conv_scan_fwd, the fused causal depthwise conv + SiLU, softplus,
discretisation, recurrence, readout, D skip and gate, through the C-ABI, carrying the conv
and SSM states from step to step.

Default workload: the 130m-shaped prefill layer (B=1, T=2048, d_inner=1536, d_state=16,
d_conv=4, f32 I/O). --config c3 runs the 2.8b-shaped layer (B=8, T=4096, d_inner=5120,
bf16 I/O); --config c2 the batched decode step (24 layers, B=64, one token per step);
--config c4 the full 24-layer 130m-shaped backbone prefill (B=4, T=2048, bf16 weights, MFMA
GEMMs), one mamba_backbone_prefill call per step; --config c4d one decode step of that
backbone for 64 sequences (after a 64-token prefill), replayed from its captured HIP graph.

Prints one JSON line. `value` is tokens/s/layer (batch tokens per step / step time);
`roofline` covers the dominant kernel call, timed with HIP events on the stream it runs
on: for prefill the call holding the scan against the VALU issue rate (the scan is
arithmetic-bound; its HBM rate is reported beside it), for the decode steps HBM, for the
backbone prefill the longest per-layer call (a GEMM against bf16 MFMA, the scan against the
VALU rate). `cpu_baseline` is the f64 CPU oracle timed on
the host on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "selective-scan prefill tokens/s/layer (d_inner=1536/5120) + HBM GB/s % peak"
# VALU issue rate: the published fp32 vector peak, 157.3 TFLOP/s, is 78.6 T fp32 FMAs/s:
# 256 CUs x 128 FMA lanes per clock x 2.4 GHz. One slot = one lane of one full-rate fp32 op.
# Plain (unpacked) fp32 ops reach this rate on gfx950: independent v_fma_f32 streams measured
# 83% of it at 16 waves per SIMD, 68% at 5.
VALU_SLOTS_PER_S = 256 * 128 * 2.4e9
# v_exp_f32 issues at quarter rate: 4 slots (measured at 3.6-4 fma slots in a mixed stream)
EXP_SLOTS = 4
# the scan's minimal slots per (t, d, n): delta*A, exp2, delta*u*B, the state fma and the
# readout fma
SCAN_SLOTS_PER_ELEMENT = 4 + EXP_SLOTS
# default warm-up steps per config, about 0.1 s of work each: from idle the GPU clock takes
# tens of milliseconds of load to ramp up (the 130m layer call measured 44 us after 20 warm-up
# steps, 40 us after 2000)
DEFAULT_WARMUP = {"c1": 2000, "c3": 100, "c2": 1000, "c5": 200, "c4": 10, "c4d": 100}
# whatever --warmup asks for, the untimed warm-up lasts at least this long: a few warm-up
# steps of a 40 us call leave the GPU clock where idle left it
MIN_WARMUP_S = 0.3


def warm_up(torch, step, n, settle=None):
    """n untimed warm-up steps (step(i), i = 0..n-1), then more untimed steps (settle(), or
    step(i) for the following i) in batches of 32 until MIN_WARMUP_S of wall time has passed
    since the first. Returns (steps run, seconds)."""
    t0 = time.perf_counter()
    for i in range(n):
        step(i)
    torch.cuda.synchronize()
    i = n
    while time.perf_counter() - t0 < MIN_WARMUP_S:
        for _ in range(32):
            if settle is None:
                step(i)
            else:
                settle()
            i += 1
        torch.cuda.synchronize()
    return i, time.perf_counter() - t0


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed steps before the timed ones (default: about 0.1 s of work for the "
                        "config; the GPU clock ramps up over the first tens of milliseconds of load)")
    p.add_argument("--config", default="c1", choices=["c1", "c3", "c2", "c4", "c4d", "c5"])
    p.add_argument("--path", default="auto", choices=["auto", "fused", "split"],
                   help="prefill: one fused mamba_conv_scan_fwd call, or mamba_conv1d_fwd then "
                        "mamba_selective_scan_fwd; auto = fused for f32 I/O, split for bf16 (where "
                        "the scan is arithmetic-bound and the conv is cheaper as its own pass)")
    p.add_argument("--event-every", type=int, default=8, metavar="E",
                   help="time the kernel calls of every E-th step of the timed region with HIP "
                        "events (the roofline's average call duration); 1 = every step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-c3", action="store_true",
                   help="with --config c1, skip the second leg that also times the 2.8b-shaped "
                        "layer (c3) and reports it under the key c3")
    p.add_argument("--no-c2", action="store_true",
                   help="with --config c1, skip the leg that also times the batched decode step "
                        "(c2) and reports it under the key c2")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="approximate CPU time budget for the oracle baseline")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                   help="only run a plain device copy of BYTES bytes a few times (the reference "
                        "kernel for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE) and exit")
    return p.parse_args(argv)


# ------------------------------------------------------------------ algorithmic bytes

def conv_bytes(s, B, T, D, K):
    """x in, u out (s bytes each), conv state read + written, taps and bias read."""
    return 2 * s * B * T * D + 8 * B * D * K + 4 * D * (K + 1)


def conv_scan_bytes(s, B, T, D, N, K):
    """The fused layer call: x, dt, z in and y out (s bytes each); B and C rows in; both
    states read and written; conv taps and bias, A_log, D and dt_bias read (u stays on chip)."""
    return (4 * s * B * T * D + 2 * s * B * T * N + 8 * B * D * (N + K) + 4 * D * (K + 1)
            + 4 * D * N + 8 * D)


def scan_bytes(s, B, T, D, N):
    """u, dt, z in and y out (s bytes each); B and C rows in; SSM state read + written;
    A_log, D and dt_bias read."""
    return 4 * s * B * T * D + 2 * s * B * T * N + 8 * B * D * N + 4 * D * N + 8 * D


def conv_step_bytes(s, L, B, D, K):
    return L * (2 * s * B * D + 8 * B * D * K + 4 * D * (K + 1))


def ssm_step_bytes(s, L, B, D, N):
    return L * (4 * s * B * D + 2 * s * B * N + 8 * B * D * N + 4 * D * N + 8 * D)


def decode_step_bytes(s, L, B, D, N, K):
    """The fused step: x, dt, z in and y out; B and C rows; both states read and written;
    conv taps and bias, A_log, D and dt_bias read (u stays on chip)."""
    return L * (4 * s * B * D + 2 * s * B * N + 8 * B * D * (N + K) + 4 * D * (K + 1) + 4 * D * N + 8 * D)


# ------------------------------------------------------------------ traffic from counters

def measured_traffic(kernel_file: str, workload: str):
    """HBM bytes per call from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source (its sha256 is recorded in the summary); else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    src = os.path.join(ROOT, "mamba_selective_scan_fwd_amd", "csrc", kernel_file)
    if not os.path.exists(path) or not os.path.exists(src):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("kernel_source_sha256") != digest:
        return None
    try:
        return float(fields["hbm_bytes_per_call"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ workloads

def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence (hip_runtime_api.h)
_hip_rt = None


def _hip():
    """The HIP runtime the process already uses (torch loads it; same soname)."""
    global _hip_rt
    if _hip_rt is None:
        import ctypes
        rt = ctypes.CDLL("libamdhip64.so.7")
        rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                           ctypes.c_void_p]
        rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip_rt = rt
    return _hip_rt


def _hip_ok(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with HIP error {rc}")


class TimingEvent:
    """A HIP event used only for timing, created with hipEventDisableSystemFence. Recording a
    default event (torch's) ends with a system-scope fence, a cache write-back and invalidate
    that stalls the GPU between the calls it brackets: at the 130m layer three such events per
    step added about 12 us to a 39 us call. Same interface as torch.cuda.Event."""

    def __init__(self):
        import ctypes
        self._ct = ctypes
        self.h = ctypes.c_void_p()
        _hip_ok(_hip().hipEventCreateWithFlags(ctypes.byref(self.h), HIP_EVENT_DISABLE_SYSTEM_FENCE),
                "hipEventCreateWithFlags")

    def record(self, stream):
        _hip_ok(_hip().hipEventRecord(self.h, self._ct.c_void_p(stream.cuda_stream)), "hipEventRecord")

    def elapsed_time(self, other):
        ms = self._ct.c_float()
        _hip_ok(_hip().hipEventElapsedTime(self._ct.byref(ms), self.h, other.h), "hipEventElapsedTime")
        return ms.value

    def __del__(self):
        if self.h:
            _hip().hipEventDestroy(self.h)


def _median(xs):
    srt = sorted(xs)
    return srt[len(srt) // 2]


def _call_events(n):
    return tuple(TimingEvent() for _ in range(n))


def _sampled_events(steps, every, n):
    """Per-call timing events for the steps i of the timed region with i % every == 0. Each
    recorded event is queue work of its own: bracketing every call of the 130m layer added
    about 4.5 us to a 36 us step, so timing every call would slow the very region whose
    throughput is reported. The sampled calls still run inside that region."""
    return {i: _call_events(n) for i in range(0, steps, max(1, every))}


def bench_prefill(args, shape):
    import numpy as np
    import torch

    import mamba_selective_scan_fwd_amd as m
    import workloads as W

    io = shape.io
    iod = torch.bfloat16 if io == "bf16" else torch.float32
    s = 2 if io == "bf16" else 4
    B, T, D, N, K = shape.B, shape.T, shape.D, shape.N, shape.K
    print(f"[bench] generating {shape.name} inputs B={B} T={T} D={D} N={N} io={io}",
          file=sys.stderr, flush=True)
    inp = W.prefill_inputs(shape)
    dev = torch.device("cuda:0")

    def up(a, as_io):
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
        return (t.to(iod) if as_io else t).to(dev)

    x, z, dt = up(inp["x"], True), up(inp["z"], True), up(inp["dt"], True)
    Bm, Cm = up(inp["Bm"], True), up(inp["Cm"], True)
    p = {k: up(inp[k], False) for k in ("conv_w", "conv_b", "dt_bias", "A_log", "D_skip")}
    conv_state = up(inp["conv_state"], False)
    ssm_state = up(inp["ssm_state"], False)
    y = torch.empty(B, T, D, dtype=iod, device=dev)
    ws = m.scan_workspace(B, T, D, N)
    stream = torch.cuda.current_stream()

    fused = args.path == "fused" or (args.path == "auto" and io == "f32")
    u = None if fused else torch.empty(B, T, D, dtype=iod, device=dev)

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        if fused:
            m.mamba_conv_scan_fwd(x, p["conv_w"], p["conv_b"], conv_state, dt, p["dt_bias"], p["A_log"],
                                  Bm, Cm, p["D_skip"], z, ssm_state, ssm_state, y, workspace=ws, stream=stream)
        else:
            m.mamba_conv1d_fwd(x, p["conv_w"], p["conv_b"], conv_state, u, stream=stream)
            if ev:
                ev[1].record(stream)
            m.mamba_selective_scan_fwd(u, dt, p["dt_bias"], p["A_log"], Bm, Cm, p["D_skip"], z,
                                       ssm_state, ssm_state, y, workspace=ws, stream=stream)
        if ev:
            ev[-1].record(stream)

    warm_steps, warm_s = warm_up(torch, lambda i: step(), args.warmup)
    print(f"[bench] warmup done ({warm_steps} steps, {warm_s:.2f} s); timing {args.steps} steps ("
          f"{'fused' if fused else 'split'} path)", file=sys.stderr, flush=True)

    # per-call events over the timed region
    evs = _sampled_events(args.steps, args.event_every, 2 if fused else 3)
    t_start, t_end = _events(torch)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs.get(i))
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    assert torch.isfinite(y.float()).all(), "non-finite output"

    ms_step = total_ms / args.steps
    tokens = B * T
    if fused:
        lb = conv_scan_bytes(s, B, T, D, N, K)
        call_ms = [e[0].elapsed_time(e[1]) for e in evs.values()]
        calls = {"mamba_conv_scan_fwd": dict(avg_ms=sum(call_ms) / len(call_ms), min_ms=min(call_ms),
                                             median_ms=_median(call_ms), bytes=lb, kernel_file="scan.hip")}
    else:
        cb, sb = conv_bytes(s, B, T, D, K), scan_bytes(s, B, T, D, N)
        lb = cb + sb
        conv_ms = [e[0].elapsed_time(e[1]) for e in evs.values()]
        scan_ms = [e[1].elapsed_time(e[2]) for e in evs.values()]
        calls = {
            "mamba_conv1d_fwd": dict(avg_ms=sum(conv_ms) / len(conv_ms), min_ms=min(conv_ms),
                                     median_ms=_median(conv_ms), bytes=cb, kernel_file="conv1d.hip"),
            "mamba_selective_scan_fwd": dict(avg_ms=sum(scan_ms) / len(scan_ms), min_ms=min(scan_ms),
                                             median_ms=_median(scan_ms), bytes=sb, kernel_file="scan.hip"),
        }
    # the call holding the scan (the longest) is arithmetic-bound: its roofline is the VALU
    # issue rate over the scan's algorithmic slots (one pass over the B*T*D*N elements)
    scan_call = "mamba_conv_scan_fwd" if fused else "mamba_selective_scan_fwd"
    traffic = measured_traffic(calls[scan_call]["kernel_file"], shape.name)
    slots = B * T * D * N * SCAN_SLOTS_PER_ELEMENT
    alu = slots / (calls[scan_call]["avg_ms"] * 1e-3) / 1e12
    result = dict(
        metric=METRIC,
        value=tokens / (ms_step * 1e-3),
        unit="tokens/s/layer",
        ms_per_step=ms_step,
        dtype="bf16" if io == "bf16" else "f32",
        config=dict(workload=f"{shape.name}: single Mamba-1 layer prefill (causal conv1d + SiLU + selective "
                             f"scan; " + ("one fused mamba_conv_scan_fwd call" if fused else
                                          "mamba_conv1d_fwd then mamba_selective_scan_fwd") +
                             f"), B={B} T={T} d_inner={D} d_state={N} d_conv={K} io={io}",
                    B=B, T=T, d_inner=D, d_state=N, d_conv=K, io_dtype=io, layer_bytes=lb,
                    path="fused" if fused else "split",
                    residency=("warm: back-to-back steps over one batch; the layer's "
                               f"{lb / 1e6:.0f} MB working set "
                               + ("fits" if lb < 200e6 else "does not fit")
                               + " the 256 MB last-level cache (MALL) between steps"
                               + ("; the same call with cold caches is under `cold`" if fused else ""))),
        roofline=dict(bound="alu", achieved=alu, peak=VALU_SLOTS_PER_S / 1e12, unit="Tslot/s",
                      frac=alu * 1e12 / VALU_SLOTS_PER_S, traffic=traffic, call=scan_call,
                      algorithmic_slots=slots, algorithmic_bytes=calls[scan_call]["bytes"],
                      avg_ms=calls[scan_call]["avg_ms"],
                      hbm_achieved_gbs=calls[scan_call]["bytes"] / (calls[scan_call]["avg_ms"] * 1e-3) / 1e9,
                      hbm_peak_gbs=HBM_PEAK_GBS,
                      hbm_frac=calls[scan_call]["bytes"] / (calls[scan_call]["avg_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS),
        calls={k: dict(avg_us=v["avg_ms"] * 1e3, median_us=v["median_ms"] * 1e3, min_us=v["min_ms"] * 1e3,
                       gbs=v["bytes"] / (v["avg_ms"] * 1e-3) / 1e9) for k, v in calls.items()},
        layer_gbs=lb / (ms_step * 1e-3) / 1e9,
    )
    result["layer_hbm_frac"] = result["layer_gbs"] / HBM_PEAK_GBS
    # the arithmetic floor of the scan (one pass over B*T*D*N elements at the VALU issue rate)
    # beside the layer's HBM floor: the one that is higher bounds the layer
    floor_s = slots / VALU_SLOTS_PER_S
    result["valu_floor_us"] = floor_s * 1e6
    result["hbm_floor_us"] = lb / (HBM_PEAK_GBS * 1e9) * 1e6
    result["valu_frac"] = floor_s / (ms_step * 1e-3)
    if fused:
        # the same call with the caches cold (the layer's 51 MB fit the 256 MB MALL)
        avg, med, mn = cold_call_times(torch, lambda: step(), stream)
        result["cold"] = dict(call=scan_call, avg_us=avg * 1e3, median_us=med * 1e3, min_us=mn * 1e3,
                              hbm_gbs=lb / (avg * 1e-3) / 1e9,
                              flush="512 MB written between repetitions, 20 repetitions")
    if B == 1:
        result["vs_step_by_step"] = step_by_step_prefill(m, torch, x, z, dt, Bm, Cm, p, conv_state,
                                                         ssm_state, stream, (128, 512, 2048))
    result["warmup_run"] = dict(steps=warm_steps, seconds=round(warm_s, 3))
    return result, inp


def second_leg_c3(args, W):
    """The 2.8b-shaped layer prefill (B=8, T=4096, d_inner=5120, bf16 I/O, conv then scan)
    timed after the default workload, in the same process, with its own warm-up; reported
    beside `value`, never in it."""
    import torch

    torch.cuda.empty_cache()
    a = argparse.Namespace(**vars(args))
    a.warmup = DEFAULT_WARMUP["c3"]
    a.steps = 50  # whatever --steps says: the leg's figure does not depend on the main line's K
    a.path = "auto"
    r, _ = bench_prefill(a, W.C3)
    torch.cuda.empty_cache()
    rl = r["roofline"]
    return dict(workload=r["config"]["workload"], steps=a.steps, warmup=a.warmup,
                warmup_run=r["warmup_run"],
                ms_per_step=r["ms_per_step"], value=r["value"], unit=r["unit"],
                calls=r["calls"], layer_gbs=r["layer_gbs"], layer_hbm_frac=r["layer_hbm_frac"],
                scan_roofline=dict(bound=rl["bound"], achieved=rl["achieved"], peak=rl["peak"],
                                   unit=rl["unit"], frac=rl["frac"], call=rl["call"],
                                   avg_ms=rl["avg_ms"], hbm_achieved_gbs=rl["hbm_achieved_gbs"],
                                   hbm_frac=rl["hbm_frac"], traffic=rl["traffic"]))


def second_leg_c2(args, W):
    """The batched decode step (24 layers x B=64, d_inner=1536) timed after the default
    workload, in the same process, with its own warm-up; reported beside `value`, never in
    it. It always times 200 steps: a step is about 70 us of GPU work, so a handful of steps
    would measure the host's enqueue of the first ones rather than the step."""
    import torch

    torch.cuda.empty_cache()
    a = argparse.Namespace(**vars(args))
    a.warmup = DEFAULT_WARMUP["c2"]
    a.steps = 200
    r, _ = bench_decode(a, W.C2)
    torch.cuda.empty_cache()
    return dict(workload=r["config"]["workload"], steps=a.steps, warmup=a.warmup,
                warmup_run=r["warmup_run"], ms_per_step=r["ms_per_step"], value=r["value"],
                unit=r["unit"], calls=r["calls"], layer_gbs=r["layer_gbs"],
                layer_hbm_frac=r["layer_hbm_frac"], roofline=r["roofline"], cold=r["cold"])


def cold_call_times(torch, fn, stream, reps=20, flush_bytes=512 << 20):
    """Call times with the caches cold: before each repetition a scratch buffer of 512 MB
    (twice the 256 MB MALL) is written, so the call's inputs come from HBM, not from the
    last-level cache where back-to-back steps of a working set this small would find them.
    Returns (avg, median, min) in ms."""
    scratch = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")
    times = []
    for r in range(reps):
        scratch.fill_(float(r))
        e0, e1 = _call_events(2)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del scratch
    srt = sorted(times)
    return sum(times) / len(times), srt[len(srt) // 2], srt[0]


def step_by_step_prefill(m, torch, x, z, dt, Bm, Cm, p, conv_state, ssm_state, stream, lengths):
    """Context for the pages' claim that the parallel prefill is 10-40x faster than a
    step-by-step prefill for T > 128 (they name no hardware): the first T tokens of the same
    B = 1 layer run as T single-token steps (one mamba_decode_step call per token, launched
    from the host, timed as a whole) against one parallel prefill call over the same T
    tokens (mamba_conv_scan_fwd, average of 20 back-to-back calls). Not part of `value`."""
    _, Tmax, D = x.shape
    K, N = conv_state.shape[-1], ssm_state.shape[-1]
    w, cb = p["conv_w"].view(1, D, K), p["conv_b"].view(1, D)
    dtb, al, ds = p["dt_bias"].view(1, D), p["A_log"].view(1, D, N), p["D_skip"].view(1, D)
    out = {}
    for T in lengths:
        if T > Tmax:
            continue
        cs = conv_state.clone().view(1, 1, D, K)
        hs = ssm_state.clone().view(1, 1, D, N)
        yt = torch.empty(1, 1, D, dtype=x.dtype, device=x.device)
        rows = [tuple(a[0, t].view(1, 1, -1) for a in (x, dt, z, Bm, Cm)) for t in range(T)]

        def run():
            for xt, dtt, zt, bt, ct in rows:
                m.mamba_decode_step(xt, w, cb, cs, dtt, dtb, al, bt, ct, ds, zt, hs, yt, stream=stream)

        run()  # warm-up pass
        torch.cuda.synchronize()
        t0, t1 = _events(torch)
        t0.record(stream)
        run()
        t1.record(stream)
        torch.cuda.synchronize()
        step_ms = t0.elapsed_time(t1)
        # the parallel prefill over the same T tokens
        xs, zs, dts, Bs, Cs = (a[:, :T].contiguous() for a in (x, z, dt, Bm, Cm))
        cs2, hs2 = conv_state.clone(), ssm_state.clone()
        ys = torch.empty_like(xs)
        ws = m.scan_workspace(1, T, D, N)

        def pre():
            m.mamba_conv_scan_fwd(xs, p["conv_w"], p["conv_b"], cs2, dts, p["dt_bias"], p["A_log"], Bs, Cs,
                                  p["D_skip"], zs, hs2, hs2, ys, workspace=ws, stream=stream)

        for _ in range(20):
            pre()
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(20):
            pre()
        t1.record(stream)
        torch.cuda.synchronize()
        pre_ms = t0.elapsed_time(t1) / 20
        out[str(T)] = dict(step_by_step_ms=step_ms, prefill_ms=pre_ms, speedup=step_ms / pre_ms)
    return dict(by_T=out, how="T mamba_decode_step calls (one token each, launched from the host) vs one "
                              "mamba_conv_scan_fwd call over the same T tokens",
                pages_claim="parallel prefill 10-40x faster than step-by-step prefill for T > 128, "
                            "no hardware stated (context only)")


def cpu_baseline_prefill(shape, inp, budget_s):
    """The f64 oracle (conv + scan) on a bounded sample of the same workload, on the host's
    cores. The oracle's C library times its own two calls (monotonic clock around the compute
    only; input conversion and the Python wrapper are outside it); each figure is the minimum
    of 3 runs. The sample is the full layer when 3 runs fit the budget, else the first D'
    channels of every batch (all T), scaled to the whole layer by D / D'. A second figure
    times one thread on a sample sized the same way."""
    import numpy as np

    from oracle import oracle

    B, T, D = shape.B, shape.T, shape.D

    def timer(dsub):
        sl = slice(0, dsub)
        return oracle.ConvScanTimer(
            inp["x"][:, :, sl], inp["conv_w"][sl], inp["conv_b"][sl], inp["conv_state"][:, sl],
            inp["dt"][:, :, sl], inp["dt_bias"][sl], inp["A_log"][sl], inp["Bm"], inp["Cm"],
            inp["D_skip"][sl], inp["z"][:, :, sl], inp["ssm_state"][:, sl], True)

    def measure(threads, share):
        probe_d = min(D, 64)
        t_probe = timer(probe_d).run(threads)
        est_full = t_probe * D / probe_d
        if 3 * est_full <= share:
            dsub = D
        else:
            dsub = max(1, min(D, int(probe_d * share / 3 / max(t_probe, 1e-6))))
        t = timer(dsub)
        best = min(t.run(threads) for _ in range(3))
        value = B * T / (best * D / dsub)
        if dsub == D:
            sample = f"full layer (B={B}, T={T}, d_inner={D}), min of 3 runs"
        else:
            sample = (f"first {dsub} of {D} channels of every batch, all T={T}, min of 3 runs; "
                      f"time scaled by {D}/{dsub}")
        return value, sample, best

    cores = oracle.threads()
    value, sample, best = measure(0, budget_s * 0.6)
    v1, s1, b1 = measure(1, budget_s * 0.4)
    return dict(value=value, unit="tokens/s/layer", cores=cores, kind="oracle", sample=sample,
                seconds=best, timing="C monotonic clock around the oracle's conv and scan calls",
                single_thread=dict(value=v1, unit="tokens/s/layer", cores=1, sample=s1, seconds=b1))


def cpu_baseline_decode(shape, budget_s):
    """The f64 oracle's decode step (conv step, then SSM step) on a bounded sample of the
    same workload: layer steps of all B sequences, timed one layer at a time on the host's
    cores, whole steps repeated while within the budget (at most 20), scaled to a step of
    L layers."""
    import numpy as np

    import workloads as W
    from oracle import oracle

    L, B = shape.L, shape.B
    P = W.decode_params(shape)
    f64 = lambda a: np.ascontiguousarray(a, dtype=np.float64)
    layers, elapsed = 0, 0.0
    while layers < 20 * L and elapsed < budget_s:  # whole steps repeated within the budget
        l = layers % L
        i = W.decode_step_inputs(shape, layers // L, layers=[l])
        cs = np.zeros((B, shape.D, shape.K))
        hs = np.zeros((B, shape.D, shape.N))
        a = {k: f64(v[0]) for k, v in i.items()}
        t0 = time.perf_counter()
        u, _ = oracle.conv1d_step(a["x"], f64(P["conv_w"][l]), f64(P["conv_b"][l]), cs)
        oracle.ssm_step(u, a["dt"], f64(P["A_log"][l]), a["Bm"], a["Cm"], f64(P["D_skip"][l]), a["z"],
                        f64(P["dt_bias"][l]), hs)
        elapsed += time.perf_counter() - t0
        layers += 1
    step_s = elapsed * L / layers
    sample = (f"{layers // L} steps of all {L} layers (B={B})" if layers % L == 0 else
              f"{layers} layer steps (B={B}), time scaled to a step of {L} layers")
    return dict(value=L * B / step_s, unit="tokens/s/layer", cores=oracle.threads(), kind="oracle",
                sample=sample, seconds=elapsed)


def bench_decode(args, shape):
    import numpy as np
    import torch

    import mamba_selective_scan_fwd_amd as m
    import workloads as W

    L, B, D, N, K = shape.L, shape.B, shape.D, shape.N, shape.K
    dev = torch.device("cuda:0")
    P = W.decode_params(shape)
    p = {k: torch.from_numpy(v).to(dev) for k, v in P.items()}
    ring = 8  # distinct per-step inputs, resident in HBM, used round-robin
    print(f"[bench] generating {ring} decode steps of inputs L={L} B={B} D={D}", file=sys.stderr, flush=True)
    steps_in = []
    for r in range(ring):
        i = W.decode_step_inputs(shape, r)
        steps_in.append({k: torch.from_numpy(v).to(dev) for k, v in i.items()})
    cs = torch.zeros(L, B, D, K, device=dev)
    hs = torch.zeros(L, B, D, N, device=dev)
    y = torch.empty(L, B, D, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        si = steps_in[i % ring]
        if ev:
            ev[0].record(stream)
        m.mamba_decode_step(si["x"], p["conv_w"], p["conv_b"], cs, si["dt"], p["dt_bias"], p["A_log"],
                            si["Bm"], si["Cm"], p["D_skip"], si["z"], hs, y, stream=stream)
        if ev:
            ev[1].record(stream)

    warm_steps, warm_s = warm_up(torch, step, args.warmup)
    evs = _sampled_events(args.steps, args.event_every, 2)
    t_start, t_end = _events(torch)
    t_start.record(stream)
    for i in range(args.steps):
        step(i, evs.get(i))
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    step_ms = [e[0].elapsed_time(e[1]) for e in evs.values()]
    ms_step = total_ms / args.steps
    sb = decode_step_bytes(4, L, B, D, N, K)
    calls = {
        "mamba_decode_step": dict(avg_ms=sum(step_ms) / len(step_ms), min_ms=min(step_ms),
                                  median_ms=_median(step_ms), bytes=sb,
                                  kernel_file="step.hip"),
    }
    dom_name = "mamba_decode_step"
    dom = calls[dom_name]
    achieved = dom["bytes"] / (dom["avg_ms"] * 1e-3) / 1e9
    result = dict(
        metric=METRIC,
        value=L * B / (ms_step * 1e-3),
        unit="tokens/s/layer",
        ms_per_step=ms_step,
        dtype="f32",
        config=dict(workload=f"{shape.name}: batched T=1 decode step (fused conv + SSM step), {L} "
                             f"independent layers in one launch, B={B} d_inner={D} d_state={N} d_conv={K} f32",
                    L=L, B=B, d_inner=D, d_state=N, d_conv=K, io_dtype="f32", step_bytes=sb),
        roofline=dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBS,
                      traffic=measured_traffic(dom["kernel_file"], shape.name), call=dom_name,
                      algorithmic_bytes=dom["bytes"], avg_ms=dom["avg_ms"]),
        calls={k: dict(avg_us=v["avg_ms"] * 1e3, median_us=v["median_ms"] * 1e3, min_us=v["min_ms"] * 1e3,
                       gbs=v["bytes"] / (v["avg_ms"] * 1e-3) / 1e9) for k, v in calls.items()},
        layer_gbs=sb / (ms_step * 1e-3) / 1e9,
    )
    result["layer_hbm_frac"] = result["layer_gbs"] / HBM_PEAK_GBS
    # the same call with the caches cold (the step's 419 MB exceed the MALL, but the states
    # of the last step may still sit in it)
    avg, med, mn = cold_call_times(torch, lambda: step(0), stream)
    result["cold"] = dict(call=dom_name, avg_us=avg * 1e3, median_us=med * 1e3, min_us=mn * 1e3,
                          hbm_gbs=sb / (avg * 1e-3) / 1e9,
                          flush="512 MB written between repetitions, 20 repetitions")
    # context: the same step as 2 L launches (conv step, then SSM step, one layer per call),
    # the per-layer launch pattern of the pages' step chain, against the one fused launch
    u = torch.empty(L, B, D, device=dev)
    lp = [{k: v[l:l + 1] for k, v in p.items()} for l in range(L)]

    def per_layer(i):
        si = steps_in[i % ring]
        for l in range(L):
            q = lp[l]
            m.mamba_conv1d_step(si["x"][l:l + 1], q["conv_w"], q["conv_b"], cs[l:l + 1], u[l:l + 1],
                                stream=stream)
            m.mamba_ssm_step(u[l:l + 1], si["dt"][l:l + 1], q["dt_bias"], q["A_log"], si["Bm"][l:l + 1],
                             si["Cm"][l:l + 1], q["D_skip"], si["z"][l:l + 1], hs[l:l + 1], y[l:l + 1],
                             stream=stream)

    for i in range(5):
        per_layer(i)
    torch.cuda.synchronize()
    reps = 20
    t0, t1 = _events(torch)
    t0.record(stream)
    for i in range(reps):
        per_layer(i)
    t1.record(stream)
    torch.cuda.synchronize()
    result["per_layer_launches"] = dict(step_us=t0.elapsed_time(t1) / reps * 1e3, launches_per_step=2 * L,
                                        fused_step_us=ms_step * 1e3,
                                        how="mamba_conv1d_step + mamba_ssm_step per layer (context)")
    result["warmup_run"] = dict(steps=warm_steps, seconds=round(warm_s, 3))
    return result, None


def m3_step_bytes(shape):
    """The Mamba-3 SISO step: per (layer, sequence, head) the SSM state read and written
    (8 hd ds), K, V and angle states read and written (8 (ds + hd + na)); per (layer,
    sequence) the in_proj row read and the output written; per layer the parameters."""
    L, B, nh, hd, ds, na = shape.L, shape.B, shape.nheads, shape.headdim, shape.d_state, shape.na
    di = nh * hd
    per_head = 8 * hd * ds + 8 * (ds + hd + na)
    per_row = 4 * shape.width + 4 * di
    per_layer = 4 * (nh + 2 * ds + 2 * nh * ds + nh + (di if shape.gate_norm else 0))
    return L * B * nh * per_head + L * B * per_row + L * per_layer


def bench_m3(args, shape):
    import torch

    import mamba_selective_scan_fwd_amd as m
    import workloads as W

    L, B = shape.L, shape.B
    dev = torch.device("cuda:0")
    P = W.m3_params(shape)
    p = {k: (None if v is None else torch.from_numpy(v).to(dev)) for k, v in P.items()}
    ring = 4  # distinct per-step in_proj rows, resident in HBM, used round-robin
    print(f"[bench] generating {ring} Mamba-3 steps of in_proj rows L={L} B={B}", file=sys.stderr, flush=True)
    rows = [torch.from_numpy(W.m3_proj(shape, step=r)).to(dev) for r in range(ring)]
    st = {k: torch.from_numpy(v).to(dev) for k, v in W.m3_states(shape).items()}
    out = torch.empty(L, B, shape.d_inner, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        if ev:
            ev[0].record(stream)
        m.mamba3_siso_step(rows[i % ring], p, shape.a_floor, st["ssm"], st["k"], st["v"], st["angle"], out,
                           shape.ngroups, shape.na, stream=stream)
        if ev:
            ev[1].record(stream)

    warm_steps, warm_s = warm_up(torch, step, args.warmup)
    evs = _sampled_events(args.steps, args.event_every, 2)
    t_start, t_end = _events(torch)
    t_start.record(stream)
    for i in range(args.steps):
        step(i, evs.get(i))
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    step_ms = [e[0].elapsed_time(e[1]) for e in evs.values()]
    ms_step = total_ms / args.steps
    sb = m3_step_bytes(shape)
    avg = sum(step_ms) / len(step_ms)
    achieved = sb / (avg * 1e-3) / 1e9
    result = dict(
        metric=METRIC,
        value=L * B / (ms_step * 1e-3),
        unit="tokens/s/layer",
        ms_per_step=ms_step,
        dtype="f32",
        config=dict(workload=f"{shape.name}: Mamba-3 SISO decode step (split, BC-norm, RoPE, trapezoidal "
                             f"update, gated norm), {L} layers in one launch, B={B}, {shape.nheads} heads x "
                             f"headdim {shape.headdim}, d_state {shape.d_state}, {shape.na} angles, f32",
                    L=L, B=B, nheads=shape.nheads, headdim=shape.headdim, d_state=shape.d_state,
                    ngroups=shape.ngroups, n_angles=shape.na, step_bytes=sb),
        roofline=dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBS, traffic=measured_traffic("mamba3.hip", shape.name),
                      call="mamba3_siso_step", algorithmic_bytes=sb, avg_ms=avg),
        calls={"mamba3_siso_step": dict(avg_us=avg * 1e3, median_us=_median(step_ms) * 1e3,
                                        min_us=min(step_ms) * 1e3,
                                        gbs=achieved)},
        layer_gbs=sb / (ms_step * 1e-3) / 1e9,
    )
    result["layer_hbm_frac"] = result["layer_gbs"] / HBM_PEAK_GBS
    result["warmup_run"] = dict(steps=warm_steps, seconds=round(warm_s, 3))
    return result, dict(P=P)


def cpu_baseline_m3(shape, data, budget_s):
    """The f64 oracle on a bounded sample of the same step: (layer, sequence) pairs, one at a
    time, until the time budget is spent; scaled to tokens/s/layer (one pair is one token of
    one layer)."""
    import time

    import numpy as np

    from oracle import mamba3 as o3
    import workloads as W

    P = data["P"]
    kw = dict(nheads=shape.nheads, headdim=shape.headdim, d_state=shape.d_state,
              ngroups=shape.ngroups, n_angles=shape.na, a_floor=shape.a_floor)
    zero = {k: v[:1, :1] for k, v in W.m3_states(W.Mamba3Shape(
        "one", L=1, B=1, nheads=shape.nheads, headdim=shape.headdim, d_state=shape.d_state,
        ngroups=shape.ngroups, n_angles=shape.n_angles)).items()}
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s and done < shape.L * shape.B:
        l, b = done % shape.L, done // shape.L
        row = W.m3_proj(shape, pairs=[(l, b)])[None]
        lp = {k: (None if v is None else v[l:l + 1]) for k, v in P.items() if k != "gate_norm_w"}
        lp["gate_w"] = None if P["gate_norm_w"] is None else P["gate_norm_w"][l:l + 1]
        o3.siso_step(row, lp, zero["ssm"], zero["k"], zero["v"], zero["angle"], **kw)
        done += 1
    dt = time.perf_counter() - t0
    return dict(value=done / dt, unit="tokens/s/layer", cores=1, kind="oracle",
                sample=f"{done} of the {shape.L * shape.B} (layer, sequence) pairs of one step, "
                       f"each through the f64 numpy oracle ({dt:.1f} s)")


def gemm_flops(M, N, K):
    return 2.0 * M * N * K


def bench_backbone(args, shape):
    """One step = one mamba_backbone_prefill call (embedding, 24 layers, norm_f, tied head).
    A second timed region runs layer 0's chain through the piece entry points (the same
    kernels the backbone call launches) with an event around every call, for the per-kernel
    breakdown and the roofline of the dominant one."""
    import numpy as np
    import torch

    import mamba_selective_scan_fwd_amd as m
    import workloads as W

    L, B, T, Dm, D, N, K, R = (shape.n_layers, shape.B, shape.T, shape.d_model, shape.D, shape.N,
                               shape.K, shape.dt_rank)
    xw = R + 2 * N
    dev = torch.device("cuda:0")
    print(f"[bench] generating {shape.name} weights and tokens (L={L} B={B} T={T})", file=sys.stderr,
          flush=True)
    w = W.backbone_weights(shape)
    tok_np = W.backbone_tokens(shape)
    bf = ("embed", "in_proj", "x_proj", "dt_proj", "out_proj")
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).to(torch.bfloat16 if k in bf else torch.float32).to(dev)
         for k, v in w.items()}
    wst = m.backbone_weights_struct(t)
    dims = m.BackboneDims(L, Dm, D, N, K, R, shape.vocab, shape.vocab_padded, shape.eps)
    tokens = torch.from_numpy(tok_np).to(dev)
    cs = torch.zeros(L, B, D, K, device=dev)
    hs = torch.zeros(L, B, D, N, device=dev)
    logits = torch.empty(B, shape.vocab, device=dev)
    ws = torch.empty(m.mamba_backbone_workspace_size(dims, B, T), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        m.mamba_backbone_prefill(dims, wst, tokens, cs, hs, logits, ws, stream=stream)

    warm_steps, warm_s = warm_up(torch, lambda i: step(), args.warmup)
    print(f"[bench] warmup done ({warm_steps} steps, {warm_s:.2f} s); timing {args.steps} steps", file=sys.stderr,
          flush=True)
    t_start, t_end = _events(torch)
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    assert torch.isfinite(logits).all(), "non-finite logits"

    # per-kernel breakdown: layer 0 through the piece entry points
    bt = B * T
    h = torch.empty(bt, Dm, device=dev)
    xn = torch.empty(bt, Dm, dtype=torch.bfloat16, device=dev)
    proj = torch.empty(bt, 2 * D, device=dev)
    u = torch.empty(B, T, D, device=dev)
    xdbl = torch.empty(bt, xw, device=dev)
    dtb = torch.empty(B, T, D, device=dev)
    y = torch.empty(B, T, D, device=dev)
    y16 = torch.zeros(bt, D, dtype=torch.bfloat16, device=dev)
    last = torch.empty(B, Dm, dtype=torch.bfloat16, device=dev)
    lg2 = torch.empty(B, shape.vocab, device=dev)
    sws = m.scan_workspace(B, T, D, N)
    xdt_n = m.mamba_xproj_dtproj_workspace_size(bt, D, R, N)
    xdt_ws = torch.empty(xdt_n, dtype=torch.uint8, device=dev) if xdt_n else None
    cs0 = torch.zeros(B, D, K, device=dev)
    hs0 = torch.zeros(B, D, N, device=dev)
    proj3 = proj.view(B, T, 2 * D)
    xdbl3 = xdbl.view(B, T, xw)
    pieces = [
        ("embed_gather", lambda: m.mamba_embed_gather(tokens, t["embed"], h, shape.vocab, stream=stream),
         None, 2 * bt * Dm + 4 * bt * Dm + 4 * bt),
        ("rmsnorm", lambda: m.mamba_rmsnorm(h, t["norm_w"][0], shape.eps, xn, stream=stream),
         None, 4 * bt * Dm + 2 * bt * Dm + 4 * Dm),
        ("gemm in_proj", lambda: m.mamba_gemm_bf16(xn, t["in_proj"][0], proj, stream=stream),
         gemm_flops(bt, 2 * D, Dm), 2 * bt * Dm + 2 * 2 * D * Dm + 4 * bt * 2 * D),
        # the conv inside x_proj's split product, then one kernel that sums its partial planes
        # and applies dt_proj
        ("conv + x_proj + dt_proj", lambda: m.mamba_conv_xproj_dtproj(
            proj3[..., :D], t["conv_w"][0], t["conv_b"][0], cs0, u, t["x_proj"][0], t["dt_proj"][0], xdbl,
            dtb.view(bt, D), workspace=xdt_ws, stream=stream),
         gemm_flops(bt, xw, D) + gemm_flops(bt, D, R),
         conv_bytes(4, B, T, D, K) + 2 * xw * D + 4 * bt * xw + 2 * D * R + 4 * bt * D),
        ("selective_scan_fwd", lambda: m.mamba_selective_scan_fwd(
            u, dtb, t["dt_bias"][0], t["A_log"][0], xdbl3[..., R:R + N], xdbl3[..., R + N:],
            t["D_skip"][0], proj3[..., D:], hs0, hs0, y, workspace=sws, stream=stream),
         None, scan_bytes(4, B, T, D, N)),
        # (the backbone's scan leaves y as bf16 for out_proj: the product reads a bf16 copy)
        ("gemm out_proj", lambda: m.mamba_gemm_bf16(y16, t["out_proj"][0], h, accumulate=True, stream=stream),
         gemm_flops(bt, Dm, D), 2 * bt * D + 2 * Dm * D + 8 * bt * Dm),
        ("gemm head", lambda: m.mamba_gemm_bf16(last, t["embed"], lg2, N=shape.vocab, stream=stream),
         gemm_flops(B, shape.vocab, Dm), 2 * shape.vocab * Dm + 2 * B * Dm + 4 * B * shape.vocab),
    ]
    reps = max(5, min(args.steps, 50))
    for _, fn, _, _ in pieces:
        fn()
    torch.cuda.synchronize()
    evs = [[_call_events(2) for _ in pieces] for _ in range(reps)]
    for r in range(reps):
        for (_, fn, _, _), (e0, e1) in zip(pieces, evs[r]):
            e0.record(stream)
            fn()
            e1.record(stream)
    torch.cuda.synchronize()
    calls = {}
    for i, (name, _, flops, nbytes) in enumerate(pieces):
        ms = [evs[r][i][0].elapsed_time(evs[r][i][1]) for r in range(reps)]
        avg = sum(ms) / len(ms)
        c = dict(avg_us=avg * 1e3, median_us=_median(ms) * 1e3, min_us=min(ms) * 1e3,
                 gbs=nbytes / (avg * 1e-3) / 1e9)
        if flops:
            c["tflops"] = flops / (avg * 1e-3) / 1e12
        calls[name] = c
    per_layer = ("rmsnorm", "gemm in_proj", "conv + x_proj + dt_proj", "selective_scan_fwd", "gemm out_proj")
    dom_name = max(per_layer, key=lambda k: calls[k]["avg_us"])
    dom = calls[dom_name]
    flops, nbytes = next((f, b) for n, _, f, b in pieces if n == dom_name)
    if flops:
        achieved = flops / (dom["avg_us"] * 1e-6) / 1e12
        roof = dict(bound="mfma", achieved=achieved, peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=achieved / MFMA_BF16_PEAK_TFLOPS, traffic=None, call=dom_name,
                    algorithmic_flops=flops, avg_ms=dom["avg_us"] * 1e-3)
    elif "scan" in dom_name:
        # the scan is arithmetic-bound, as in the single-layer prefill: VALU issue rate over
        # one pass of B*T*D*N elements, with its HBM rate beside it
        slots = B * T * D * N * SCAN_SLOTS_PER_ELEMENT
        achieved = slots / (dom["avg_us"] * 1e-6) / 1e12
        hbm = nbytes / (dom["avg_us"] * 1e-6) / 1e9
        roof = dict(bound="alu", achieved=achieved, peak=VALU_SLOTS_PER_S / 1e12, unit="Tslot/s",
                    frac=achieved * 1e12 / VALU_SLOTS_PER_S,
                    traffic=measured_traffic("scan.hip", shape.name), call=dom_name,
                    algorithmic_slots=slots, algorithmic_bytes=nbytes, avg_ms=dom["avg_us"] * 1e-3,
                    hbm_achieved_gbs=hbm, hbm_peak_gbs=HBM_PEAK_GBS, hbm_frac=hbm / HBM_PEAK_GBS)
    else:
        achieved = nbytes / (dom["avg_us"] * 1e-6) / 1e9
        roof = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=achieved / HBM_PEAK_GBS, traffic=measured_traffic("conv1d.hip", shape.name),
                    call=dom_name, algorithmic_bytes=nbytes, avg_ms=dom["avg_us"] * 1e-3)
    layer_us = sum(calls[k]["avg_us"] for k in per_layer)
    result = dict(
        metric=METRIC,
        value=B * T * L / (ms_step * 1e-3),
        unit="tokens/s/layer",
        ms_per_step=ms_step,
        dtype="bf16",
        config=dict(workload=f"{shape.name}: full {L}-layer Mamba-1 backbone prefill (embedding, RMSNorm, "
                             f"in_proj/x_proj/dt_proj/out_proj bf16 MFMA GEMMs, conv1d, scan, residual, "
                             f"norm_f, tied {shape.vocab}-vocab head), B={B} T={T} d_model={Dm} "
                             f"d_inner={D} d_state={N} dt_rank={R}",
                    B=B, T=T, n_layers=L, d_model=Dm, d_inner=D, d_state=N, d_conv=K, dt_rank=R,
                    vocab=shape.vocab),
        roofline=roof,
        calls=calls,
        backbone_tokens_per_s=B * T / (ms_step * 1e-3),
        layer_chain_us=layer_us,
        layer_gbs=None,
        layer_hbm_frac=None,
    )
    result["warmup_run"] = dict(steps=warm_steps, seconds=round(warm_s, 3))
    return result, dict(weights=w, tokens=tok_np)


def bench_backbone_decode(args, shape):
    """One step = one replay of the captured backbone decode step (one token for each of B
    sequences through all layers and the head). Eager (one launch per kernel) is timed too."""
    import numpy as np
    import torch

    import mamba_selective_scan_fwd_amd as m
    import workloads as W

    B, P = 64, 64  # sequences, prefill length before the timed decode steps
    L, Dm, D, N, K, R = shape.n_layers, shape.d_model, shape.D, shape.N, shape.K, shape.dt_rank
    dev = torch.device("cuda:0")
    print(f"[bench] generating backbone weights (L={L}) and {B} x {P} prompt tokens", file=sys.stderr, flush=True)
    w = W.backbone_weights(shape)
    bs = W.BackboneShape("c4d", n_layers=L, B=B, T=P + args.steps + args.warmup + 8)
    tok = torch.from_numpy(W.backbone_tokens(bs)).to(dev)
    bf = ("embed", "in_proj", "x_proj", "dt_proj", "out_proj")
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).to(torch.bfloat16 if k in bf else torch.float32).to(dev)
         for k, v in w.items()}
    wst = m.backbone_weights_struct(t)
    dims = m.BackboneDims(L, Dm, D, N, K, R, shape.vocab, shape.vocab_padded, shape.eps)
    cs = torch.zeros(L, B, D, K, device=dev)
    hs = torch.zeros(L, B, D, N, device=dev)
    logits = torch.empty(B, shape.vocab, device=dev)
    ws = torch.empty(m.mamba_backbone_workspace_size(dims, B, P), dtype=torch.uint8, device=dev)
    m.mamba_backbone_prefill(dims, wst, tok[:, :P].contiguous(), cs, hs, logits, ws)
    wsd = torch.empty(m.mamba_backbone_decode_workspace_size(dims, B), dtype=torch.uint8, device=dev)
    step_tok = torch.empty(B, dtype=torch.int32, device=dev)
    graph = m.DecodeGraph(dims, wst, step_tok, cs, hs, logits, wsd)
    stream = torch.cuda.current_stream()
    pos = [P]

    def next_tokens():
        step_tok.copy_(tok[:, pos[0]])
        pos[0] += 1

    def warm(i):
        next_tokens()
        graph.launch(stream)

    # beyond the counted warm-up steps the graph replays on the same tokens (the token buffer
    # holds only the counted steps)
    warm_steps, warm_s = warm_up(torch, warm, args.warmup, settle=lambda: graph.launch(stream))
    t0, t1 = _events(torch)
    t0.record(stream)
    for _ in range(args.steps):
        next_tokens()
        graph.launch(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_graph = t0.elapsed_time(t1) / args.steps
    # eager, for context (same number of steps, states keep advancing)
    e0, e1 = _events(torch)
    e0.record(stream)
    for _ in range(min(args.steps, 8)):
        m.mamba_backbone_decode_step(dims, wst, step_tok, cs, hs, logits, wsd, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / min(args.steps, 8)
    assert torch.isfinite(logits).all(), "non-finite logits"
    graph.close()
    # the step is weight-streaming bound: every layer's projections and the head are read once
    wbytes = 2 * (L * (2 * D * Dm + (R + 2 * N) * D + D * R + Dm * D) + shape.vocab * Dm)
    sbytes = 8 * L * B * D * (N + K)
    nbytes = wbytes + sbytes
    achieved = nbytes / (ms_graph * 1e-3) / 1e9
    result = dict(
        metric=METRIC,
        value=B * L / (ms_graph * 1e-3),
        unit="tokens/s/layer",
        ms_per_step=ms_graph,
        dtype="bf16",
        config=dict(workload=f"c4d: one decode step of the {L}-layer 130m-shaped backbone for B={B} sequences "
                             f"(after a {P}-token prefill), replayed from its captured HIP graph",
                    B=B, n_layers=L, d_model=Dm, d_inner=D, d_state=N, vocab=shape.vocab),
        roofline=dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBS, traffic=None, call="decode step (graph)",
                      algorithmic_bytes=nbytes, avg_ms=ms_graph),
        calls={"graph replay": dict(avg_us=ms_graph * 1e3), "eager step": dict(avg_us=ms_eager * 1e3)},
        backbone_tokens_per_s=B / (ms_graph * 1e-3),
        layer_gbs=None,
        layer_hbm_frac=None,
    )
    result["warmup_run"] = dict(steps=warm_steps, seconds=round(warm_s, 3))
    return result, None


def cpu_baseline_backbone(shape, data, budget_s):
    """The f64 backbone oracle on sequence 0 of the batch over its first T' tokens, all layers
    (T' from a probe so the run takes about budget_s)."""
    from oracle import backbone as ob
    from oracle import oracle

    w, tok = data["weights"], data["tokens"]
    L = shape.n_layers

    def run(tp):
        t0 = time.perf_counter()
        ob.prefill(w, tok[:1, :tp], L, shape.D, shape.N, shape.dt_rank, shape.vocab, shape.eps)
        return time.perf_counter() - t0

    probe = min(shape.T, 64)
    t_probe = run(probe)
    tp = max(probe, min(shape.T, int(probe * budget_s / max(t_probe, 1e-6))))
    elapsed = run(tp) if tp != probe else t_probe
    return dict(value=tp * L / elapsed, unit="tokens/s/layer", cores=oracle.threads(), kind="oracle",
                sample=f"sequence 0 of {shape.B}, first {tp} of {shape.T} tokens, all {L} layers and the head",
                seconds=elapsed)


def main(argv=None):
    args = parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs the hot path on one GPU only; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported. The work shards across GPUs by batch or "
              "d_inner with no communication; run one process per GPU on its own share.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        n = args.calibrate_copy // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps(dict(calibrate_copy_bytes=n * 4, launches=3)), flush=True)
        return
    if args.warmup is None:
        args.warmup = DEFAULT_WARMUP[args.config]
    shape = W.CONFIGS.get(args.config, W.C4)
    if args.config == "c2":
        result, inp = bench_decode(args, shape)
    elif args.config == "c4":
        result, inp = bench_backbone(args, shape)
    elif args.config == "c4d":
        result, inp = bench_backbone_decode(args, W.C4)
    elif args.config == "c5":
        result, inp = bench_m3(args, shape)
    else:
        result, inp = bench_prefill(args, shape)
    c3 = c2 = None
    if args.config == "c1" and not args.no_c3:
        c3 = second_leg_c3(args, W)
    if args.config == "c1" and not args.no_c2:
        c2 = second_leg_c2(args, W)
    cpu = None
    if not args.no_cpu_baseline and (inp is not None or args.config == "c2"):
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        if args.config == "c4":
            cpu = cpu_baseline_backbone(shape, inp, args.cpu_seconds)
        elif args.config == "c2":
            cpu = cpu_baseline_decode(shape, args.cpu_seconds)
        elif args.config == "c5":
            cpu = cpu_baseline_m3(shape, inp, args.cpu_seconds)
        else:
            cpu = cpu_baseline_prefill(shape, inp, args.cpu_seconds)
    line = dict(
        metric=result["metric"], value=result["value"], unit=result["unit"], n_gpus=1,
        steps=args.steps, warmup=args.warmup, ms_per_step=result["ms_per_step"],
        higher_is_better=True, scaling="weak", vs_baseline=None, dtype=result["dtype"],
        data="synthetic", config=result["config"], roofline=result["roofline"],
        cpu_baseline=cpu, calls=result["calls"], layer_gbs=result["layer_gbs"],
        layer_hbm_frac=result["layer_hbm_frac"])
    for extra in ("backbone_tokens_per_s", "layer_chain_us", "valu_floor_us", "hbm_floor_us", "valu_frac",
                  "vs_step_by_step", "cold", "per_layer_launches", "warmup_run"):
        if extra in result:
            line[extra] = result[extra]
    if c3 is not None:
        line["c3"] = c3
    if c2 is not None:
        line["c2"] = c2
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
