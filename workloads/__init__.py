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
  c5  Mamba-3 SISO decode step, L=24 B=64, 24 heads x headdim 64, d_state 128, 1 group,
      64 RoPE angles, gated output norm (130m-shaped: d_model 768, d_inner 1536)

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
M3_PROJ, M3_PARAMS, M3_STATE = 20, 21, 22


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


@dataclasses.dataclass(frozen=True)
class Mamba3Shape:
    name: str
    L: int
    B: int
    nheads: int
    headdim: int
    d_state: int
    ngroups: int = 1
    n_angles: int = -1  # -1: d_state / 2 (every pair rotated)
    a_floor: float = 1e-4
    gate_norm: bool = True
    d_model: int = 0  # shape label only

    @property
    def na(self) -> int:
        return self.d_state // 2 if self.n_angles < 0 else self.n_angles

    @property
    def d_inner(self) -> int:
        return self.nheads * self.headdim

    @property
    def width(self) -> int:
        """in_proj row width: z | x | B | C | dt | A | trap | angles."""
        return 2 * self.d_inner + 2 * self.ngroups * self.d_state + 3 * self.nheads + self.na


C5 = Mamba3Shape("c5", L=24, B=64, nheads=24, headdim=64, d_state=128, d_model=768)
CONFIGS = {"c0": C0, "c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5}
CONFIG_INDEX = {"c0": 0, "c1": 1, "c2": 2, "c3": 3, "c4": 4, "c5": 5}


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


# ------------------------------------------------------- Mamba-3 SISO step (c5) inputs
#
# in_proj rows: z, x, B, C ~ N(0, 1); dt_raw ~ N(0, 0.1^2); a_raw ~ N(1, 1) (softplus around
# 1.3); trap_raw ~ N(0, 1) (lambda mostly in 0.15 .. 0.85); angles ~ N(0, 1). Parameters:
# dt_bias as Mamba-1 (inverse softplus of a log-uniform [1e-3, 0.1] draw, per head);
# B/C norm weights and the gate-norm weight 1 + N(0, 0.1^2); B/C biases 1 + N(0, 0.1^2)
# (Mamba-3 starts them at one); D ~ U(0.5, 1.5). States zero unless drawn (N(0, 1); angles
# U(-pi, pi)).

def m3_params(shape: Mamba3Shape, seed: int = 0, cfg: int = 5) -> dict:
    L, nh, ds, di = shape.L, shape.nheads, shape.d_state, shape.d_inner
    g = rng(seed, cfg, M3_PARAMS)
    p = dict(
        dt_bias=np.stack([dt_bias_init(nh, rng(seed, cfg, DT0, l))[0] for l in range(L)]),
        b_norm_w=(1.0 + normal(g, (L, ds), 0.1)).astype(np.float32),
        c_norm_w=(1.0 + normal(g, (L, ds), 0.1)).astype(np.float32),
        b_bias=(1.0 + normal(g, (L, nh, ds), 0.1)).astype(np.float32),
        c_bias=(1.0 + normal(g, (L, nh, ds), 0.1)).astype(np.float32),
        D=g.uniform(0.5, 1.5, size=(L, nh)).astype(np.float32),
        gate_norm_w=(1.0 + normal(g, (L, di), 0.1)).astype(np.float32) if shape.gate_norm else None,
    )
    return p


def m3_proj(shape: Mamba3Shape, step: int = 0, seed: int = 0, cfg: int = 5, pairs=None) -> np.ndarray:
    """in_proj rows [L, B, W] of one step (or only the listed (l, b) rows, [len(pairs), W])."""
    di, gs, nh, na = shape.d_inner, shape.ngroups * shape.d_state, shape.nheads, shape.na
    todo = pairs if pairs is not None else [(l, b) for l in range(shape.L) for b in range(shape.B)]
    rows = np.empty((len(todo), shape.width), np.float32)
    for r, (l, b) in enumerate(todo):
        g = rng(seed, cfg, M3_PROJ, l * 100003 + b, step)
        rows[r, :2 * di + 2 * gs] = normal(g, 2 * di + 2 * gs)
        o = 2 * di + 2 * gs
        rows[r, o:o + nh] = normal(g, nh, 0.1)
        rows[r, o + nh:o + 2 * nh] = 1.0 + normal(g, nh)
        rows[r, o + 2 * nh:o + 3 * nh] = normal(g, nh)
        rows[r, o + 3 * nh:] = normal(g, na)
    return rows if pairs is not None else rows.reshape(shape.L, shape.B, shape.width)


def m3_states(shape: Mamba3Shape, seed: int = 0, cfg: int = 5, random: bool = False) -> dict:
    """ssm [L, B, nh, hd, ds], k [L, B, nh, ds], v [L, B, nh, hd], angle [L, B, nh, max(na, 1)]."""
    L, B, nh, hd, ds = shape.L, shape.B, shape.nheads, shape.headdim, shape.d_state
    na1 = max(shape.na, 1)
    shapes = dict(ssm=(L, B, nh, hd, ds), k=(L, B, nh, ds), v=(L, B, nh, hd), angle=(L, B, nh, na1))
    if not random:
        return {k: np.zeros(v, np.float32) for k, v in shapes.items()}
    g = rng(seed, cfg, M3_STATE)
    out = {k: normal(g, v) for k, v in shapes.items() if k != "angle"}
    out["angle"] = g.uniform(-np.pi, np.pi, size=shapes["angle"]).astype(np.float32)
    return out
