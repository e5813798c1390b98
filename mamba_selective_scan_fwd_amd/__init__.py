"""Python binding of the gfx950 Mamba-1 selective-scan C-ABI (include/mamba_ssm.h).

The functions carry the C names and only marshal arguments: device pointers and the
current HIP stream come from torch tensors, and every step of the computation runs in
the HIP kernels of libmamba_ssm.so. There is no fallback: if the library is missing or
a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "MambaError", "MAMBA_F32", "MAMBA_BF16", "library_path", "load_library", "symbols",
    "mamba_version", "mamba_last_error", "mamba_conv1d_fwd", "mamba_selective_scan_fwd",
    "mamba_selective_scan_workspace_size", "mamba_conv1d_step", "mamba_ssm_step",
    "scan_workspace", "mamba_embed_gather", "mamba_rmsnorm", "mamba_gemm_bf16",
    "mamba_xproj_dtproj_workspace_size", "mamba_xproj_dtproj", "mamba_conv_xproj_dtproj",
    "BackboneDims", "BackboneWeights", "mamba_backbone_workspace_size", "mamba_backbone_prefill",
    "Mamba3SisoParams", "mamba3_siso_step",
]

MAMBA_F32 = 0
MAMBA_BF16 = 1

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libmamba_ssm.so")

# exported symbol -> (argtypes, restype)
_P, _I, _I64, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
symbols = {
    "mamba_last_error": ([], ctypes.c_char_p),
    "mamba_version": ([], ctypes.c_char_p),
    "mamba_conv1d_fwd": ([_P, _I64, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P], _I),
    "mamba_selective_scan_workspace_size": ([_I, _I, _I, _I], _SZ),
    "mamba_selective_scan_fwd": ([_P, _P, _P, _I, _P, _P, _P, _I64, _P, _P, _I64, _P, _P, _P,
                                  _I, _I, _I, _I, _I, _P, _SZ, _P], _I),
    "mamba_conv1d_step": ([_P, _I64, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P], _I),
    "mamba_ssm_step": ([_P, _P, _P, _I, _P, _P, _P, _I64, _P, _P, _I64, _P, _P, _I, _I, _I,
                        _I, _I, _P], _I),
    "mamba_conv_scan_fwd": ([_P, _I64, _P, _P, _P, _P, _P, _I, _P, _P, _P, _I64, _P, _P, _I64, _P, _P,
                             _P, _P, _I, _I, _I, _I, _I, _I, _P, _SZ, _P], _I),
    "mamba_conv_scan_fwd_noalloc": ([_P, _I64, _P, _P, _P, _P, _P, _I, _P, _P, _P, _I64, _P, _P, _I64,
                                     _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P], _I),
    "mamba_decode_step": ([_P, _I64, _P, _P, _P, _P, _P, _I, _P, _P, _P, _I64, _P, _P, _I64, _P, _P,
                           _P, _I, _I, _I, _I, _I, _I, _P], _I),
    "mamba_embed_gather": ([_P, _P, _P, _I64, _I, _I, _P], _I),
    "mamba_rmsnorm": ([_P, _I64, _P, ctypes.c_float, _P, _I, _I64, _I, _P], _I),
    "mamba_gemm_bf16": ([_P, _I, _I64, _P, _I64, _P, _I64, _I, _I, _I, _I, _P], _I),
    "mamba_xproj_dtproj_workspace_size": ([_I, _I, _I, _I], _SZ),
    "mamba_xproj_dtproj": ([_P, _I64, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _SZ, _P], _I),
    "mamba_conv_xproj_dtproj": ([_P, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                 _P, _SZ, _P], _I),
    "mamba_backbone_workspace_size": ([_P, _I, _I], _SZ),
    "mamba_backbone_prefill": ([_P, _P, _P, _I, _I, _P, _P, _P, _P, _SZ, _P], _I),
    "mamba_backbone_prefill_ex": ([_P, _P, _P, _I, _I, _P, _P, _P, _SZ, _P], _I),
    "mamba_backbone_decode_workspace_size": ([_P, _I], _SZ),
    "mamba_backbone_decode_step": ([_P, _P, _P, _I, _P, _P, _P, _P, _SZ, _P], _I),
    "mamba_backbone_decode_graph_create": ([_P, _P, _P, _I, _P, _P, _P, _P, _SZ,
                                            ctypes.POINTER(ctypes.c_void_p)], _I),
    "mamba_graph_launch": ([_P, _P], _I),
    "mamba_graph_destroy": ([_P], None),
    "mamba3_siso_step": ([_P, _I64, _P, ctypes.c_float, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                          _I, _P], _I),
}


class BackboneDims(ctypes.Structure):
    """mamba_backbone_dims."""
    _fields_ = [("n_layers", ctypes.c_int), ("d_model", ctypes.c_int), ("d_inner", ctypes.c_int),
                ("d_state", ctypes.c_int), ("d_conv", ctypes.c_int), ("dt_rank", ctypes.c_int),
                ("vocab", ctypes.c_int), ("vocab_padded", ctypes.c_int), ("eps", ctypes.c_float)]


class BackboneWeights(ctypes.Structure):
    """mamba_backbone_weights: device pointers of the layer-stacked weights."""
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "embed", "norm_f", "norm_w", "in_proj", "conv_w", "conv_b", "x_proj", "dt_proj",
        "dt_bias", "A_log", "D_skip", "out_proj")]

class Mamba3SisoParams(ctypes.Structure):
    """mamba3_siso_params: device pointers of the layer-stacked Mamba-3 parameters."""
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "dt_bias", "b_norm_w", "c_norm_w", "b_bias", "c_bias", "D", "gate_norm_w")]


class PrefillIO(ctypes.Structure):
    """mamba_prefill_io."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("tokens", "embeds", "lengths", "logits", "hidden")]


_STATUS = {1: "MAMBA_EINVAL", 2: "MAMBA_EUNSUPPORTED", 3: "MAMBA_EWORKSPACE", 4: "MAMBA_EHIP"}


class MambaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libmamba_ssm.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError(f"{library_path} is not built; run __graft_entry__.build() or "
                              "python -m mamba_selective_scan_fwd_amd._build")
        lib = ctypes.CDLL(library_path)
        for name, (argtypes, restype) in symbols.items():
            f = getattr(lib, name)
            f.argtypes = argtypes
            f.restype = restype
        _lib = lib
    return _lib


def mamba_version() -> str:
    return load_library().mamba_version().decode()


def mamba_last_error() -> str:
    return load_library().mamba_last_error().decode()


def _check(status: int) -> None:
    if status != 0:
        raise MambaError(status, mamba_last_error())


# ------------------------------------------------------------------ marshalling helpers

def _ptr(t):
    """Device pointer of a tensor, or NULL for None. Plain ints pass through (raw pointers)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _io_dtype(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return MAMBA_F32
    if t.dtype == torch.bfloat16:
        return MAMBA_BF16
    raise TypeError(f"unsupported I/O dtype {t.dtype} (float32 or bfloat16)")


def _row_stride(t, name: str) -> int:
    """Row stride of a 3-D [outer, inner, width] view whose rows (outer, inner) are evenly
    spaced: element (o, i, w) at (o * inner + i) * stride + w."""
    if t.dim() != 3:
        raise ValueError(f"{name} must be 3-D")
    o, i, w = t.shape
    if w > 1 and t.stride(2) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    if i > 1:
        rs = t.stride(1)
        if o > 1 and t.stride(0) != i * rs:
            raise ValueError(f"{name}: rows must be evenly spaced (stride(0) == shape[1] * stride(1))")
        return rs
    if o > 1:
        return t.stride(0)
    return max(w, 1)


# --------------------------------------------------------------------------- the calls

def mamba_conv1d_fwd(x, conv_w, conv_b, conv_state, u, stream=None) -> None:
    """Prefill conv1d + SiLU. x: [B, T, >=D] view (last dim contiguous, rows may be wider,
    e.g. the x lane of an in_proj output); conv_w [D, K] f32; conv_b [D] f32 or None;
    conv_state [B, D, K] f32 (updated in place) or None; u [B, T, D] out."""
    Bsz, T = x.shape[0], x.shape[1]
    D, K = conv_w.shape
    xs = _row_stride(x, "x")
    _check(load_library().mamba_conv1d_fwd(
        _ptr(x), xs, _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(u), _io_dtype(u),
        Bsz, T, D, K, _stream(stream)))


def mamba_selective_scan_workspace_size(B: int, T: int, D: int, N: int) -> int:
    return int(load_library().mamba_selective_scan_workspace_size(B, T, D, N))


def scan_workspace(B: int, T: int, D: int, N: int, device="cuda"):
    """A device buffer large enough for mamba_selective_scan_fwd at this shape (or None)."""
    import torch
    n = mamba_selective_scan_workspace_size(B, T, D, N)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def mamba_selective_scan_fwd(u, dt, dt_bias, A_log, Bm, Cm, D_skip, z, ssm_state_in,
                             ssm_state_out, y, delta_softplus=True, workspace=None,
                             stream=None) -> None:
    """Prefill selective scan. u, dt, y: [B, T, D] contiguous; Bm, Cm: [B, T, >=N] views
    sharing one row stride; z: [B, T, >=D] view or None; A_log [D, N]; dt_bias, D_skip [D]
    or None; states [B, D, N] f32 (in may be None; out may be None or equal to in).
    workspace: a uint8 device tensor of mamba_selective_scan_workspace_size bytes."""
    Bsz, T, D = u.shape
    N = A_log.shape[1]
    bcs = _row_stride(Bm, "Bm")
    if _row_stride(Cm, "Cm") != bcs:
        raise ValueError("Bm and Cm must share one row stride")
    zs = _row_stride(z, "z") if z is not None else 0
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().mamba_selective_scan_fwd(
        _ptr(u), _ptr(dt), _ptr(dt_bias), int(bool(delta_softplus)), _ptr(A_log), _ptr(Bm),
        _ptr(Cm), bcs, _ptr(D_skip), _ptr(z), zs, _ptr(ssm_state_in), _ptr(ssm_state_out),
        _ptr(y), _io_dtype(u), Bsz, T, D, N, _ptr(workspace), ws_bytes, _stream(stream)))


def mamba_conv_scan_fwd(x, conv_w, conv_b, conv_state, dt, dt_bias, A_log, Bm, Cm, D_skip, z,
                        ssm_state_in, ssm_state_out, y, u=None, workspace=None, delta_softplus=True,
                        stream=None) -> None:
    """Fused conv + scan prefill. x: [B, T, >=D] view (row-strided lane allowed); conv_w
    [D, K]; conv_state [B, D, K] or None; other arguments as mamba_selective_scan_fwd; u:
    optional [B, T, D] output."""
    Bsz, T, D = y.shape
    K = conv_w.shape[1]
    N = A_log.shape[1]
    xs = _row_stride(x, "x")
    bcs = _row_stride(Bm, "Bm")
    if _row_stride(Cm, "Cm") != bcs:
        raise ValueError("Bm and Cm must share one row stride")
    zs = _row_stride(z, "z") if z is not None else 0
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().mamba_conv_scan_fwd(
        _ptr(x), xs, _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(dt), _ptr(dt_bias),
        int(bool(delta_softplus)), _ptr(A_log), _ptr(Bm), _ptr(Cm), bcs, _ptr(D_skip), _ptr(z), zs,
        _ptr(ssm_state_in), _ptr(ssm_state_out), _ptr(u), _ptr(y), _io_dtype(y), Bsz, T, D, K, N,
        _ptr(workspace), wsb, _stream(stream)))


def mamba_conv_scan_fwd_noalloc(x, conv_w, conv_b, conv_state, dt, dt_bias, A_log, Bm, Cm, D_skip, z,
                                ssm_state_in, ssm_state_out, y, u=None, delta_softplus=True,
                                stream=None) -> None:
    """mamba_conv_scan_fwd without a workspace: the library's fixed scratch stands in for it.
    Arguments as mamba_conv_scan_fwd."""
    Bsz, T, D = y.shape
    K = conv_w.shape[1]
    N = A_log.shape[1]
    xs = _row_stride(x, "x")
    bcs = _row_stride(Bm, "Bm")
    if _row_stride(Cm, "Cm") != bcs:
        raise ValueError("Bm and Cm must share one row stride")
    zs = _row_stride(z, "z") if z is not None else 0
    _check(load_library().mamba_conv_scan_fwd_noalloc(
        _ptr(x), xs, _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(dt), _ptr(dt_bias),
        int(bool(delta_softplus)), _ptr(A_log), _ptr(Bm), _ptr(Cm), bcs, _ptr(D_skip), _ptr(z), zs,
        _ptr(ssm_state_in), _ptr(ssm_state_out), _ptr(u), _ptr(y), _io_dtype(y), Bsz, T, D, K, N,
        _stream(stream)))


def mamba_conv1d_step(x, conv_w, conv_b, conv_state, u, stream=None) -> None:
    """Decode conv step for L layers. x: [L, B, >=D] view; conv_w [L, D, K]; conv_b [L, D]
    or None; conv_state [L, B, D, K] (in place); u [L, B, D]."""
    L, Bsz = u.shape[0], u.shape[1]
    _, D, K = conv_w.shape
    xs = _row_stride(x, "x")
    _check(load_library().mamba_conv1d_step(
        _ptr(x), xs, _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(u), _io_dtype(u),
        L, Bsz, D, K, _stream(stream)))


def mamba_ssm_step(u, dt, dt_bias, A_log, Bm, Cm, D_skip, z, ssm_state, y,
                   delta_softplus=True, stream=None) -> None:
    """Decode SSM step for L layers. u, dt, y: [L, B, D]; Bm, Cm: [L, B, >=N] views sharing
    one row stride; z: [L, B, >=D] view or None; A_log [L, D, N]; dt_bias, D_skip [L, D] or
    None; ssm_state [L, B, D, N] (in place)."""
    L, Bsz, D = u.shape
    N = A_log.shape[2]
    bcs = _row_stride(Bm, "Bm")
    if _row_stride(Cm, "Cm") != bcs:
        raise ValueError("Bm and Cm must share one row stride")
    zs = _row_stride(z, "z") if z is not None else 0
    _check(load_library().mamba_ssm_step(
        _ptr(u), _ptr(dt), _ptr(dt_bias), int(bool(delta_softplus)), _ptr(A_log), _ptr(Bm),
        _ptr(Cm), bcs, _ptr(D_skip), _ptr(z), zs, _ptr(ssm_state), _ptr(y), _io_dtype(u), L, Bsz,
        D, N, _stream(stream)))


def mamba_decode_step(x, conv_w, conv_b, conv_state, dt, dt_bias, A_log, Bm, Cm, D_skip, z,
                      ssm_state, y, u=None, delta_softplus=True, stream=None) -> None:
    """Fused conv step + SSM step for L layers. x, dt, z: [L, B, D] (x and z may be row-strided
    lanes); Bm, Cm: [L, B, >=N] rows; conv_state [L, B, D, K]; ssm_state [L, B, D, N]."""
    L, Bsz, D = y.shape
    K = conv_state.shape[-1]
    N = ssm_state.shape[-1]
    xs = _row_stride(x, "x")
    bcs = _row_stride(Bm, "Bm")
    if _row_stride(Cm, "Cm") != bcs:
        raise ValueError("Bm and Cm must share a row stride")
    zs = _row_stride(z, "z") if z is not None else 0
    _check(load_library().mamba_decode_step(
        _ptr(x), xs, _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(dt), _ptr(dt_bias),
        int(bool(delta_softplus)), _ptr(A_log), _ptr(Bm), _ptr(Cm), bcs, _ptr(D_skip), _ptr(z), zs,
        _ptr(ssm_state), _ptr(u), _ptr(y), _io_dtype(y), L, Bsz, D, K, N, _stream(stream)))


# ------------------------------------------------------------------ backbone pieces

def mamba_embed_gather(tokens, E, out, vocab, stream=None) -> None:
    """out[r, :] = E[tokens[r], :]. tokens int32 [rows]; E bf16 [>= vocab, d_model]; out f32."""
    rows = tokens.numel()
    _check(load_library().mamba_embed_gather(_ptr(tokens), _ptr(E), _ptr(out), rows, vocab,
                                             E.shape[1], _stream(stream)))


def mamba_rmsnorm(x, w, eps, out, rows=None, x_row_stride=None, stream=None) -> None:
    """RMSNorm of `rows` rows of x (row stride x_row_stride, default contiguous) into out
    (f32 or bf16, [rows, d_model] contiguous)."""
    d_model = out.shape[-1]
    rows = out.numel() // d_model if rows is None else rows
    xs = d_model if x_row_stride is None else x_row_stride
    _check(load_library().mamba_rmsnorm(_ptr(x), xs, _ptr(w), float(eps), _ptr(out), _io_dtype(out),
                                        rows, d_model, _stream(stream)))


def mamba_gemm_bf16(A, W, C, accumulate=False, M=None, N=None, K=None, lda=None, ldw=None,
                    ldc=None, stream=None) -> None:
    """C[M, N] (+)= A[M, K] @ W[N, K]^T with bf16 operands and f32 accumulation."""
    M = A.shape[0] if M is None else M
    K = W.shape[1] if K is None else K
    N = W.shape[0] if N is None else N
    lda = A.stride(0) if lda is None else lda
    ldw = W.stride(0) if ldw is None else ldw
    ldc = C.stride(0) if ldc is None else ldc
    _check(load_library().mamba_gemm_bf16(_ptr(A), _io_dtype(A), lda, _ptr(W), ldw, _ptr(C), ldc, M,
                                          N, K, int(bool(accumulate)), _stream(stream)))


def mamba_xproj_dtproj_workspace_size(M: int, d_inner: int, dt_rank: int, d_state: int) -> int:
    return int(load_library().mamba_xproj_dtproj_workspace_size(M, d_inner, dt_rank, d_state))


def mamba_xproj_dtproj(u, W_x, W_dt, xdbl, dt, dt_bias=None, delta_softplus=False, workspace=None, M=None,
                       ldu=None, stream=None) -> None:
    """xdbl = u @ W_x^T and dt = xdbl[:, :dt_rank] @ W_dt^T (bf16 operands, f32 sums), then
    dt + dt_bias and softplus when given (the scan's delta). u: [M, >= d_inner] f32 rows;
    W_x [dt_rank + 2 d_state, d_inner] and W_dt [d_inner, dt_rank] bf16; xdbl
    [M, dt_rank + 2 d_state] and dt [M, d_inner] f32; dt_bias [d_inner] f32 or None;
    workspace a device buffer of mamba_xproj_dtproj_workspace_size bytes, or None (allocated
    here when needed)."""
    import torch
    d_inner, dt_rank = W_dt.shape
    d_state = (W_x.shape[0] - dt_rank) // 2
    M = u.shape[0] if M is None else M
    ldu = u.stride(0) if ldu is None else ldu
    need = mamba_xproj_dtproj_workspace_size(M, d_inner, dt_rank, d_state)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=u.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().mamba_xproj_dtproj(_ptr(u), ldu, _ptr(W_x), _ptr(W_dt), _ptr(xdbl), _ptr(dt),
                                             _ptr(dt_bias), int(bool(delta_softplus)), M, d_inner, dt_rank,
                                             d_state, _ptr(workspace), nbytes, _stream(stream)))


def mamba_conv_xproj_dtproj(x, conv_w, conv_b, conv_state, u, W_x, W_dt, xdbl, dt, lengths=None,
                            dt_bias=None, delta_softplus=False, workspace=None, stream=None) -> None:
    """u = silu(conv(x)) (conv state carried), xdbl = u @ W_x^T, dt = xdbl[:, :dt_rank] @ W_dt^T
    (then + dt_bias and softplus when given, as mamba_xproj_dtproj).
    x: [B, T, >= d_inner] f32 view (row stride as it is); conv_w [d_inner, d_conv]; conv_b
    [d_inner] or None; conv_state [B, d_inner, d_conv] or None; u [B, T, d_inner]; W_x, W_dt
    bf16; xdbl [B*T, dt_rank + 2 d_state]; dt [B*T, d_inner]; lengths [B] int32 or None."""
    import torch
    B, T = x.shape[0], x.shape[1]
    d_inner, d_conv = conv_w.shape
    dt_rank = W_dt.shape[1]
    d_state = (W_x.shape[0] - dt_rank) // 2
    need = mamba_xproj_dtproj_workspace_size(B * T, d_inner, dt_rank, d_state)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().mamba_conv_xproj_dtproj(
        _ptr(x), _row_stride(x, "x"), _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(lengths), _ptr(u),
        _ptr(W_x), _ptr(W_dt), _ptr(xdbl), _ptr(dt), _ptr(dt_bias), int(bool(delta_softplus)), B, T, d_inner,
        d_conv, dt_rank, d_state, _ptr(workspace), nbytes, _stream(stream)))


def mamba_backbone_workspace_size(dims: BackboneDims, B: int, T: int) -> int:
    return int(load_library().mamba_backbone_workspace_size(ctypes.byref(dims), B, T))


def mamba_backbone_prefill(dims: BackboneDims, weights: BackboneWeights, tokens, conv_state,
                           ssm_state, logits, workspace, stream=None) -> None:
    """Prefill B prompts of T tokens through the whole backbone; logits of each last token."""
    Bsz, T = tokens.shape
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().mamba_backbone_prefill(
        ctypes.byref(dims), ctypes.byref(weights), _ptr(tokens), Bsz, T, _ptr(conv_state),
        _ptr(ssm_state), _ptr(logits), _ptr(workspace), ws_bytes, _stream(stream)))


_BACKBONE_BF16 = ("embed", "in_proj", "x_proj", "dt_proj", "out_proj")


def backbone_weights_struct(t: dict) -> BackboneWeights:
    """Build the mamba_backbone_weights struct from a dict of contiguous device tensors (bf16
    for the embedding and the projections, f32 for the rest). The caller keeps the tensors
    alive while the struct is in use."""
    import torch
    w = BackboneWeights()
    for name, _ in BackboneWeights._fields_:
        x = t[name]
        want = torch.bfloat16 if name in _BACKBONE_BF16 else torch.float32
        if x.dtype != want or not x.is_contiguous() or not x.is_cuda:
            raise ValueError(f"backbone weight {name}: need a contiguous device {want} tensor")
        setattr(w, name, x.data_ptr())
    return w


def mamba_backbone_decode_workspace_size(dims: BackboneDims, B: int) -> int:
    return int(load_library().mamba_backbone_decode_workspace_size(ctypes.byref(dims), B))


def mamba_backbone_decode_step(dims: BackboneDims, weights: BackboneWeights, tokens, conv_state,
                               ssm_state, logits, workspace, stream=None) -> None:
    """One decode step of the whole backbone: tokens [B] int32 -> logits [B, vocab]; states in
    place."""
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().mamba_backbone_decode_step(
        ctypes.byref(dims), ctypes.byref(weights), _ptr(tokens), tokens.numel(), _ptr(conv_state),
        _ptr(ssm_state), _ptr(logits), _ptr(workspace), ws_bytes, _stream(stream)))


class DecodeGraph:
    """The backbone decode step captured into a HIP graph (mamba_backbone_decode_graph_create).
    The buffers given here are baked in: write the next tokens into `tokens`, then launch()."""

    def __init__(self, dims: BackboneDims, weights: BackboneWeights, tokens, conv_state, ssm_state,
                 logits, workspace):
        self._keep = (dims, weights, tokens, conv_state, ssm_state, logits, workspace)
        handle = ctypes.c_void_p()
        ws_bytes = workspace.numel() * workspace.element_size()
        _check(load_library().mamba_backbone_decode_graph_create(
            ctypes.byref(dims), ctypes.byref(weights), _ptr(tokens), tokens.numel(), _ptr(conv_state),
            _ptr(ssm_state), _ptr(logits), _ptr(workspace), ws_bytes, ctypes.byref(handle)))
        self._h = handle

    def launch(self, stream=None) -> None:
        _check(load_library().mamba_graph_launch(self._h, _stream(stream)))

    def close(self) -> None:
        if self._h:
            load_library().mamba_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def mamba_backbone_prefill_ex(dims: BackboneDims, weights: BackboneWeights, B: int, T: int, conv_state,
                              ssm_state, workspace, tokens=None, embeds=None, lengths=None, logits=None,
                              hidden=None, stream=None) -> None:
    """Prefill variants: token ids [B, T] or raw input rows embeds [B, T, d_model]; optional
    per-sequence lengths [B] int32 (right-padded ragged batch); logits [B, vocab] of each last
    valid token and/or hidden [B, T, d_model] (norm_f at every position)."""
    io = PrefillIO(_ptr(tokens), _ptr(embeds), _ptr(lengths), _ptr(logits), _ptr(hidden))
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().mamba_backbone_prefill_ex(
        ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(io), B, T, _ptr(conv_state),
        _ptr(ssm_state), _ptr(workspace), ws_bytes, _stream(stream)))


# ------------------------------------------------------------ Mamba-3 SISO decode step

def mamba3_siso_step(proj, params: dict, a_floor: float, ssm_state, k_state, v_state, angle_state,
                     out, ngroups: int, n_angles: int, stream=None) -> None:
    """Phases F3-F7 of the Mamba-3 SISO step for L layers and B sequences. proj [L, B, >= W]
    (rows may be strided); params: dict of f32 tensors dt_bias [L, nh], b_norm_w / c_norm_w
    [L, ds], b_bias / c_bias [L, nh, ds], D [L, nh], gate_norm_w [L, nh * hd] or None;
    ssm_state [L, B, nh, hd, ds], k_state [L, B, nh, ds], v_state [L, B, nh, hd],
    angle_state [L, B, nh, max(na, 1)]; out [L, B, nh * hd]."""
    L, Bsz, nh, hd, ds = ssm_state.shape
    c = Mamba3SisoParams(*[_ptr(params.get(n)) for n in (
        "dt_bias", "b_norm_w", "c_norm_w", "b_bias", "c_bias", "D", "gate_norm_w")])
    _check(load_library().mamba3_siso_step(
        _ptr(proj), _row_stride(proj, "proj"), ctypes.byref(c), float(a_floor), _ptr(ssm_state),
        _ptr(k_state), _ptr(v_state), _ptr(angle_state), _ptr(out), L, Bsz, nh, hd, ds, ngroups,
        n_angles, _stream(stream)))
