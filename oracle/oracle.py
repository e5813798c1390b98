"""Python front end of the f64 CPU oracle (oracle/mamba_oracle.c).

TEST INFRASTRUCTURE. Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no code
with the HIP library and never imports it.

Every array is converted to contiguous float64 before the call, so the oracle
reads f32 and bf16-rounded inputs exactly. Shapes and meanings follow the C file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mamba_oracle.c")
_LIB = os.path.join(_HERE, "libmamba_oracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain IEEE f64: no -ffast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
            "-Wall", "-Wextra", "-Werror", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None
_lib_path = None


def use_library(path: str | None) -> None:
    """Point the wrappers at another build of the oracle source (None: the default).
    Used by the mutation test, which compiles copies with planted mistakes."""
    global _lib, _lib_path
    _lib, _lib_path = None, path


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = _lib_path or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        I64 = ctypes.c_int64
        L.oracle_conv1d_fwd.argtypes = [P, I64, P, P, P, P, I, I, I, I]
        L.oracle_conv1d_fwd.restype = None
        L.oracle_selective_scan_fwd.argtypes = [P, P, P, I, P, P, P, I64, P, P, I64, P, P, P,
                                                I, I, I, I]
        L.oracle_selective_scan_fwd.restype = None
        L.oracle_conv1d_step.argtypes = [P, I64, P, P, P, P, I, I, I]
        L.oracle_conv1d_step.restype = None
        L.oracle_ssm_step.argtypes = [P, P, P, I, P, P, P, I64, P, P, I64, P, P, I, I, I]
        L.oracle_ssm_step.restype = None
        L.oracle_softplus.argtypes = [ctypes.c_double]
        L.oracle_softplus.restype = ctypes.c_double
        L.oracle_silu.argtypes = [ctypes.c_double]
        L.oracle_silu.restype = ctypes.c_double
        L.oracle_threads.argtypes = []
        L.oracle_threads.restype = ctypes.c_int
        L.oracle_time_conv_scan.argtypes = [P, I64, P, P, P, P, P, P, I, P, P, P, I64, P, P, I64,
                                            P, P, P, I, I, I, I, I, I]
        L.oracle_time_conv_scan.restype = ctypes.c_double
        _lib = L
    return _lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def threads() -> int:
    """OpenMP threads the oracle's channel loops use."""
    return int(lib().oracle_threads())


def softplus(v: float) -> float:
    return lib().oracle_softplus(float(v))


def silu(v: float) -> float:
    return lib().oracle_silu(float(v))


def conv1d_fwd(x, conv_w, conv_b=None, conv_state=None):
    """Prefill conv + SiLU.

    x: [B, T, D] (or [B, T, row] with the channel lane in columns 0..D-1 -- pass the
    full rows and D is taken from conv_w); conv_w: [D, K]; conv_b: [D] or None;
    conv_state: [B, D, K] or None (zero history).
    Returns (u [B,T,D] f64, conv_state_out [B,D,K] f64 or None).
    """
    x = _f64(x)
    w = _f64(conv_w)
    D, K = w.shape
    Bsz, T, row = x.shape
    assert row >= D
    bias = _f64(conv_b)
    st = None if conv_state is None else _f64(conv_state).copy()
    u = np.zeros((Bsz, T, D), np.float64)
    lib().oracle_conv1d_fwd(_p(x), row, _p(w), _p(bias), _p(st), _p(u), Bsz, T, D, K)
    return u, st


def selective_scan_fwd(u, dt, A_log, Bm, Cm, D_skip=None, z=None, dt_bias=None,
                       delta_softplus=True, ssm_state=None):
    """Prefill selective scan.

    u, dt: [B, T, D]; A_log: [D, N]; Bm, Cm: [B, T, row] with n in columns 0..N-1
    (both share one row length); D_skip, dt_bias: [D] or None; z: [B, T, zrow] with
    the gate in columns 0..D-1, or None; ssm_state: [B, D, N] or None (zeros).
    Returns (y [B,T,D] f64, ssm_state_out [B,D,N] f64).
    """
    u = _f64(u)
    dt = _f64(dt)
    A = _f64(A_log)
    D, N = A.shape
    Bsz, T, Du = u.shape
    assert Du == D and dt.shape == u.shape
    Bm = _f64(Bm)
    Cm = _f64(Cm)
    assert Bm.shape == Cm.shape and Bm.shape[:2] == (Bsz, T) and Bm.shape[2] >= N
    zz = _f64(z)
    zrow = 0
    if zz is not None:
        assert zz.shape[:2] == (Bsz, T) and zz.shape[2] >= D
        zrow = zz.shape[2]
    st_in = None if ssm_state is None else _f64(ssm_state)
    st_out = np.zeros((Bsz, D, N), np.float64)
    y = np.zeros((Bsz, T, D), np.float64)
    lib().oracle_selective_scan_fwd(_p(u), _p(dt), _p(_f64(dt_bias)), int(bool(delta_softplus)),
                                    _p(A), _p(Bm), _p(Cm), Bm.shape[2], _p(_f64(D_skip)),
                                    _p(zz), zrow, _p(st_in), _p(st_out), _p(y), Bsz, T, D, N)
    return y, st_out


def conv1d_step(x, conv_w, conv_b, conv_state):
    """One decode step of the conv for one layer. x: [B, row] (lane in cols 0..D-1);
    conv_w [D,K]; conv_b [D] or None; conv_state [B,D,K]. Returns (u [B,D], new state)."""
    x = _f64(x)
    w = _f64(conv_w)
    D, K = w.shape
    Bsz, row = x.shape
    st = _f64(conv_state).copy()
    u = np.zeros((Bsz, D), np.float64)
    lib().oracle_conv1d_step(_p(x), row, _p(w), _p(_f64(conv_b)), _p(st), _p(u), Bsz, D, K)
    return u, st


def ssm_step(u, dt, A_log, Bm, Cm, D_skip, z, dt_bias, ssm_state, delta_softplus=True):
    """One decode step of the SSM for one layer. u, dt: [B, D]; Bm, Cm: [B, row];
    z: [B, zrow] or None; ssm_state [B,D,N]. Returns (y [B,D], new state)."""
    u = _f64(u)
    dt = _f64(dt)
    A = _f64(A_log)
    D, N = A.shape
    Bsz = u.shape[0]
    Bm = _f64(Bm)
    Cm = _f64(Cm)
    zz = _f64(z)
    zrow = 0 if zz is None else zz.shape[1]
    st = _f64(ssm_state).copy()
    y = np.zeros((Bsz, D), np.float64)
    lib().oracle_ssm_step(_p(u), _p(dt), _p(_f64(dt_bias)), int(bool(delta_softplus)), _p(A),
                          _p(Bm), _p(Cm), Bm.shape[1], _p(_f64(D_skip)), _p(zz), zrow, _p(st),
                          _p(y), Bsz, D, N)
    return y, st


class ConvScanTimer:
    """CPU-baseline timing of the prefill layer (conv + SiLU, then the scan) on fixed inputs.

    The inputs are converted to contiguous f64 once, here; each ``run`` calls the C timing
    entry, which times only the two oracle calls with the monotonic clock, on ``threads``
    OpenMP threads (0: the default team). Arguments follow conv1d_fwd and selective_scan_fwd;
    x carries the channel lane in columns 0..D-1 of its rows, Bm and Cm share one row length.
    """

    def __init__(self, x, conv_w, conv_b, conv_state, dt, dt_bias, A_log, Bm, Cm, D_skip, z,
                 ssm_state=None, delta_softplus=True):
        self.x = _f64(x)
        self.w = _f64(conv_w)
        self.D, self.K = self.w.shape
        self.B, self.T, self.xrow = self.x.shape
        self.conv_b = _f64(conv_b)
        self.st0 = None if conv_state is None else _f64(conv_state)
        self.dt = _f64(dt)
        self.dt_bias = _f64(dt_bias)
        self.A = _f64(A_log)
        self.N = self.A.shape[1]
        self.Bm = _f64(Bm)
        self.Cm = _f64(Cm)
        self.D_skip = _f64(D_skip)
        self.z = _f64(z)
        self.zrow = 0 if self.z is None else self.z.shape[2]
        self.h0 = None if ssm_state is None else _f64(ssm_state)
        self.softplus = int(bool(delta_softplus))
        self.u = np.zeros((self.B, self.T, self.D), np.float64)
        self.y = np.zeros((self.B, self.T, self.D), np.float64)
        self.h1 = np.zeros((self.B, self.D, self.N), np.float64)

    def run(self, threads: int = 0) -> float:
        """One timed pass; returns the seconds the two oracle calls took."""
        st = None if self.st0 is None else self.st0.copy()
        return float(lib().oracle_time_conv_scan(
            _p(self.x), self.xrow, _p(self.w), _p(self.conv_b), _p(st), _p(self.u), _p(self.dt),
            _p(self.dt_bias), self.softplus, _p(self.A), _p(self.Bm), _p(self.Cm),
            self.Bm.shape[2], _p(self.D_skip), _p(self.z), self.zrow, _p(self.h0), _p(self.h1),
            _p(self.y), self.B, self.T, self.D, self.N, self.K, int(threads)))

