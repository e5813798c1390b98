"""Seeded synthetic inputs for the selective-scan hot path.

This module is shared by the tests, the bench and the smoke check, and feeds both
the HIP library and the CPU oracle. It holds no arithmetic of the method itself:
only shapes, random draws, the parameter-initialisation recipe and bf16 rounding
of stored inputs.

Workloads (one Mamba-1 layer unless stated):
  c0  B=1  T=32    D=64    N=16 K=4  f32          (tiny correctness case)
  c1  B=1  T=2048  D=1536  N=16 K=4  f32          (130m-shaped prefill layer)
  c2  L=24 B=64    D=1536  N=16 K=4  f32, T=1 x 1000 decode steps
  c3  B=8  T=4096  D=5120  N=16 K=4  bf16 I/O     (2.8b-shaped prefill layer)
  c4  24-layer 130m-shaped backbone, B=4, T=2048, d_model 768, vocab 50280

Distributions: x, z, B, C ~ N(0, 1); dt_raw ~ N(0, 0.1^2); dt_bias is the inverse
softplus of dt0 with dt0 log-uniform in [1e-3, 0.1]; A_log[d, n] = log(n + 1)
(S4D-real); D = 1; conv_w ~ U(-0.5, 0.5); conv_b = 0; zero initial states.
Each tensor draws from its own stream, keyed by (seed, workload, tensor, layer, step).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# tensor ids for the per-tensor random streams
X, Z, BM, CM, DT, DT0, CONVW = 0, 1, 2, 3, 4, 5, 6
ALOG_RAND, DSKIP_RAND, CONVB_RAND, STATE_RAND = 7, 8, 9, 16
EMBED, W_IN, W_X, W_DT, W_OUT, TOKENS = 10, 11, 12, 13, 14, 15


@dataclasses.dataclass(frozen=True)
class PrefillShape:
    name: str
    B: int
    T: int
    D: int
    N: int = 16
    K: int = 4
    io: str = "f32"  # "f32" or "bf16"
    d_model: int = 0  # shape label only for the single-layer workloads
    dt_rank: int = 0  # shape label only


@dataclasses.dataclass(frozen=True)
class DecodeShape:
    name: str
    L: int
    B: int
    D: int
    N: int = 16
    K: int = 4
    steps: int = 1000
    io: str = "f32"


@dataclasses.dataclass(frozen=True)
class BackboneShape:
    name: str
    n_layers: int = 24
    B: int = 4
    T: int = 2048
    d_model: int = 768
    D: int = 1536
    N: int = 16
    K: int = 4
    dt_rank: int = 48
    vocab: int = 50280
    vocab_padded: int = 50304
    eps: float = 1e-5


C0 = PrefillShape("c0", B=1, T=32, D=64)
C1 = PrefillShape("c1", B=1, T=2048, D=1536, d_model=768, dt_rank=48)
C2 = DecodeShape("c2", L=24, B=64, D=1536)
C3 = PrefillShape("c3", B=8, T=4096, D=5120, io="bf16", d_model=2560, dt_rank=160)
C4 = BackboneShape("c4")
CONFIGS = {"c0": C0, "c1": C1, "c2": C2, "c3": C3, "c4": C4}
CONFIG_INDEX = {"c0": 0, "c1": 1, "c2": 2, "c3": 3, "c4": 4}


def rng(seed: int, cfg: int, tensor: int, layer: int = 0, step: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg, tensor, layer, step])))


# ---------------------------------------------------------------- bf16 storage

def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round f32 values to the nearest bf16 (ties to even); returns f32 holding bf16 values.
    NaN stays NaN (quiet)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(a)
    out = (rounded & 0xFFFFFFFF).astype(np.uint32).view(np.float32).copy()
    if nan.any():
        out[nan] = np.float32("nan")
    return out


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns of f32 values that are already bf16-exact."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


_TORCH_ROUND_MIN = 1 << 20


def store(a: np.ndarray, io: str) -> np.ndarray:
    """The value a tensor holds once stored in the I/O dtype (f32 array either way).
    Large arrays are rounded with torch's CPU bf16 conversion, which is the same
    round-to-nearest-even (checked against bf16_round in the tests), only faster."""
    a = np.asarray(a, dtype=np.float32)
    if io != "bf16":
        return a
    if a.size >= _TORCH_ROUND_MIN:
        try:
            import torch
        except ImportError:
            return bf16_round(a)
        return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(torch.float32).numpy()
    return bf16_round(a)


# ------------------------------------------------------- parameter init recipe

def inv_softplus(v: np.ndarray) -> np.ndarray:
    """y with log(1 + exp(y)) = v, in f64: y = v + log(-expm1(-v))."""
    v = np.asarray(v, dtype=np.float64)
    return v + np.log(-np.expm1(-v))


def dt_bias_init(D: int, g: np.random.Generator, dt_min=1e-3, dt_max=0.1):
    """dt0 log-uniform in [dt_min, dt_max]; bias = inverse softplus of dt0 (f64 -> f32).
    Returns (bias f32 [D], dt0 f64 [D])."""
    dt0 = np.exp(g.uniform(math.log(dt_min), math.log(dt_max), size=D))
    return inv_softplus(dt0).astype(np.float32), dt0


def s4d_real_alog(D: int, N: int) -> np.ndarray:
    return np.log(np.tile(np.arange(1, N + 1, dtype=np.float64), (D, 1))).astype(np.float32)


# ------------------------------------------------------------ prefill inputs

def layer_params(D: int, N: int, K: int, seed: int, cfg: int, layer: int = 0,
                 random_alog: bool = False, random_extras: bool = False) -> dict:
    """Per-layer parameters (all f32). random_alog draws A_log with no structure
    (log of U(0.5, 16)); random_extras also draws D_skip and conv_b."""
    bias, dt0 = dt_bias_init(D, rng(seed, cfg, DT0, layer))
    if random_alog:
        A_log = np.log(rng(seed, cfg, ALOG_RAND, layer).uniform(0.5, 16.0, size=(D, N))).astype(np.float32)
    else:
        A_log = s4d_real_alog(D, N)
    conv_w = rng(seed, cfg, CONVW, layer).uniform(-0.5, 0.5, size=(D, K)).astype(np.float32)
    if random_extras:
        D_skip = rng(seed, cfg, DSKIP_RAND, layer).uniform(0.5, 1.5, size=D).astype(np.float32)
        conv_b = rng(seed, cfg, CONVB_RAND, layer).uniform(-0.2, 0.2, size=D).astype(np.float32)
    else:
        D_skip = np.ones(D, np.float32)
        conv_b = np.zeros(D, np.float32)
    return dict(dt_bias=bias, dt0=dt0, A_log=A_log, D_skip=D_skip, conv_w=conv_w, conv_b=conv_b)


def normal(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    out = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def prefill_inputs(shape: PrefillShape, seed: int = 0, cfg: int | None = None, layer: int = 0,
                   random_alog: bool = False, random_extras: bool = False,
                   random_state: bool = False) -> dict:
    """All inputs of one prefill layer as f32 numpy arrays holding the stored values
    (bf16-rounded where the I/O dtype is bf16).
    x, z, dt: [B,T,D]; Bm, Cm: [B,T,N]; conv_state: [B,D,K]; ssm_state: [B,D,N]."""
    if cfg is None:
        cfg = CONFIG_INDEX.get(shape.name, 99)
    B, T, D, N, K = shape.B, shape.T, shape.D, shape.N, shape.K
    p = layer_params(D, N, K, seed, cfg, layer, random_alog, random_extras)
    io = shape.io
    inp = dict(
        x=store(normal(rng(seed, cfg, X, layer), (B, T, D)), io),
        z=store(normal(rng(seed, cfg, Z, layer), (B, T, D)), io),
        Bm=store(normal(rng(seed, cfg, BM, layer), (B, T, N)), io),
        Cm=store(normal(rng(seed, cfg, CM, layer), (B, T, N)), io),
        dt=store(normal(rng(seed, cfg, DT, layer), (B, T, D), std=0.1), io),
        conv_state=np.zeros((B, D, K), np.float32),
        ssm_state=np.zeros((B, D, N), np.float32),
    )
    if random_state:
        g = rng(seed, cfg, STATE_RAND, layer)
        inp["conv_state"] = normal(g, (B, D, K))
        inp["ssm_state"] = normal(g, (B, D, N))
    inp.update(p)
    return inp


def decode_params(shape: DecodeShape, seed: int = 0, cfg: int = 2) -> dict:
    """Stacked per-layer parameters for the decode workload: [L, D], [L, D, N], [L, D, K]."""
    ps = [layer_params(shape.D, shape.N, shape.K, seed, cfg, l) for l in range(shape.L)]
    return {k: np.stack([p[k] for p in ps]) for k in ("dt_bias", "A_log", "D_skip", "conv_w", "conv_b")}


def decode_step_inputs(shape: DecodeShape, step: int, seed: int = 0, cfg: int = 2,
                       layers=None) -> dict:
    """Host-side inputs of one decode step (all layers, or the listed layers):
    x, z, dt [L', B, D]; Bm, Cm [L', B, N]."""
    layers = range(shape.L) if layers is None else layers
    out = {k: [] for k in ("x", "z", "dt", "Bm", "Cm")}
    for l in layers:
        out["x"].append(normal(rng(seed, cfg, X, l, step), (shape.B, shape.D)))
        out["z"].append(normal(rng(seed, cfg, Z, l, step), (shape.B, shape.D)))
        out["dt"].append(normal(rng(seed, cfg, DT, l, step), (shape.B, shape.D), std=0.1))
        out["Bm"].append(normal(rng(seed, cfg, BM, l, step), (shape.B, shape.N)))
        out["Cm"].append(normal(rng(seed, cfg, CM, l, step), (shape.B, shape.N)))
    return {k: store(np.stack(v), shape.io) for k, v in out.items()}


# --------------------------------------------------- device-side decode inputs

def torch_generator(seed: int, cfg: int, tensor: int, layer: int = 0, step: int = 0, device="cuda"):
    """A torch generator on `device` keyed like rng(): for inputs too large to draw on the host
    (1000 decode steps x 24 layers). Deterministic for a given torch build and device type."""
    import torch

    key = int(np.random.SeedSequence([seed, cfg, tensor, layer, step]).generate_state(1, np.uint64)[0])
    g = torch.Generator(device=device)
    g.manual_seed(key & ((1 << 63) - 1))
    return g


def decode_step_inputs_torch(shape: DecodeShape, step: int, seed: int = 0, cfg: int = 2,
                             device="cuda") -> dict:
    """Per-step decode inputs drawn on the device: x, z, dt [L,B,D]; Bm, Cm [L,B,N] (f32,
    same distributions as decode_step_inputs, different streams)."""
    import torch

    L, B, D, N = shape.L, shape.B, shape.D, shape.N
    out = {}
    for name, tid, shp, std in (("x", X, (L, B, D), 1.0), ("z", Z, (L, B, D), 1.0),
                                ("dt", DT, (L, B, D), 0.1), ("Bm", BM, (L, B, N), 1.0),
                                ("Cm", CM, (L, B, N), 1.0)):
        g = torch_generator(seed, cfg, tid, 0, step, device)
        t = torch.randn(shp, generator=g, device=device, dtype=torch.float32)
        out[name] = t * std if std != 1.0 else t
    if shape.io == "bf16":
        out = {k: v.to(torch.bfloat16) for k, v in out.items()}
    return out


# ------------------------------------------------------------ backbone (c4) weights

def backbone_weights(shape: BackboneShape, seed: int = 0, cfg: int = 4) -> dict:
    """Random-init weights of the Mamba-1 backbone (host, numpy f32; bf16 weights hold
    bf16-exact values). Embedding and projections ~ N(0, 0.02^2) stored bf16 (nn.Linear layout
    [out, in]; the embedding is [vocab_padded, d_model] with zero padding rows); SSM parameters
    as in the single-layer workloads; norm weights 1."""
    L, Dm, D, N, K, R = shape.n_layers, shape.d_model, shape.D, shape.N, shape.K, shape.dt_rank
    def w(tid, layer, shp):
        return store(normal(rng(seed, cfg, tid, layer), shp, std=0.02), "bf16")
    embed = np.zeros((shape.vocab_padded, Dm), np.float32)
    embed[:shape.vocab] = w(EMBED, 0, (shape.vocab, Dm))
    out = dict(embed=embed, norm_f=np.ones(Dm, np.float32), norm_w=np.ones((L, Dm), np.float32),
               in_proj=np.stack([w(W_IN, l, (2 * D, Dm)) for l in range(L)]),
               x_proj=np.stack([w(W_X, l, (R + 2 * N, D)) for l in range(L)]),
               dt_proj=np.stack([w(W_DT, l, (D, R)) for l in range(L)]),
               out_proj=np.stack([w(W_OUT, l, (Dm, D)) for l in range(L)]))
    ps = [layer_params(D, N, K, seed, cfg, l) for l in range(L)]
    for k in ("conv_w", "conv_b", "dt_bias", "A_log", "D_skip"):
        out[k] = np.stack([p[k] for p in ps])
    return out


def backbone_tokens(shape: BackboneShape, seed: int = 0, cfg: int = 4) -> np.ndarray:
    """Token ids uniform in [0, vocab), [B, T] int32."""
    return rng(seed, cfg, TOKENS).integers(0, shape.vocab, size=(shape.B, shape.T)).astype(np.int32)
