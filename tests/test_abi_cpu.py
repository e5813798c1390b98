"""The C-ABI library on the CPU: it loads, exports every symbol include/mamba_ssm.h declares,
and rejects bad arguments before touching the GPU (validation runs before any HIP call).
No compute call is made here."""
import ctypes
import os
import re

import pytest

import mamba_selective_scan_fwd_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mamba_ssm.h")

F32, BF16 = m.MAMBA_F32, m.MAMBA_BF16
EINVAL, EUNSUP, EWS = 1, 2, 3
FAKE = 0x7F0000000000  # a well-aligned address; never dereferenced (calls fail validation first)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mamba3?_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = m.load_library()
    names = declared_functions()
    assert {"mamba_conv1d_fwd", "mamba_selective_scan_fwd", "mamba_conv1d_step",
            "mamba_ssm_step", "mamba_last_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in mamba_ssm.h but not exported"
    assert set(names) == set(m.symbols), "binding symbol table and header disagree"


def test_version_and_empty_error():
    assert "gfx950" in m.mamba_version()


def scan_call(**kw):
    a = dict(u=FAKE, dt=FAKE, dt_bias=None, sp=1, A_log=FAKE, Bm=FAKE, Cm=FAKE, bcs=16, D_skip=None,
             z=None, zs=0, si=None, so=None, y=FAKE + (1 << 30), io=F32, B=1, T=32, D=64, N=16,
             ws=FAKE + (1 << 35), wsb=1 << 20, stream=None)
    a.update(kw)
    st = m.load_library().mamba_selective_scan_fwd(
        a["u"], a["dt"], a["dt_bias"], a["sp"], a["A_log"], a["Bm"], a["Cm"], a["bcs"], a["D_skip"],
        a["z"], a["zs"], a["si"], a["so"], a["y"], a["io"], a["B"], a["T"], a["D"], a["N"], a["ws"],
        a["wsb"], a["stream"])
    return st, m.mamba_last_error()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(u=None), EINVAL, "u is NULL"),
    (dict(N=0), EINVAL, "N = 0"),
    (dict(N=65), EUNSUP, "N = 65"),
    (dict(T=-1), EINVAL, "T = -1"),
    (dict(io=7), EINVAL, "io_dtype"),
    (dict(bcs=8), EINVAL, "bc_row_stride"),
    (dict(z=FAKE + (1 << 31), zs=10), EINVAL, "z_row_stride"),
    (dict(u=FAKE + 2), EINVAL, "aligned"),
    (dict(so=FAKE + 64), EINVAL, "ssm_state_out overlaps u"),
    (dict(y=FAKE), EINVAL, "y overlaps u"),
    (dict(B=1, T=2048, D=1536, ws=None, wsb=0), EWS, "workspace"),
])
def test_scan_validation(kw, status, needle):
    st, msg = scan_call(**kw)
    assert st == status, msg
    assert needle in msg and msg.startswith("mamba_selective_scan_fwd")


def test_scan_workspace_too_small_and_misaligned():
    need = m.mamba_selective_scan_workspace_size(1, 2048, 1536, 16)
    assert need > 0
    st, msg = scan_call(B=1, T=2048, D=1536, ws=FAKE + (1 << 34), wsb=need - 1)
    assert st == EWS and "workspace_bytes" in msg
    st, msg = scan_call(B=1, T=2048, D=1536, ws=FAKE + (1 << 34) + 4, wsb=need)
    assert st == EINVAL and "256-byte" in msg


def test_scan_empty_batch_is_noop():
    st, msg = scan_call(u=None, dt=None, A_log=None, Bm=None, Cm=None, y=None, B=0, ws=None)
    assert st == 0, msg
    st, msg = scan_call(u=None, dt=None, A_log=None, Bm=None, Cm=None, y=None, D=0)
    assert st == 0, msg


def test_scan_state_partial_overlap_rejected():
    st, msg = scan_call(si=FAKE + (1 << 33), so=FAKE + (1 << 33) + 64)
    assert st == EINVAL and "ssm_state_out overlaps ssm_state_in" in msg


def test_workspace_size_formula():
    # one chunk (no carry) needs no workspace; the large shapes need one
    assert m.mamba_selective_scan_workspace_size(1, 32, 64, 16) >= 0
    assert m.mamba_selective_scan_workspace_size(8, 4096, 5120, 16) % 256 == 0
    assert m.mamba_selective_scan_workspace_size(0, 32, 64, 16) == 0
    # a long sequence over few channels: the chunk count stops at its cap of 64 (longer chunks
    # instead), so the workspace is 64 chunk sums and end states per channel, the carried SSM
    # state and the carried conv state (8 slots), each rounded up to 256 bytes
    def capped(B, D, N, chunks=64):
        a = lambda n: (n + 255) // 256 * 256
        return a(4 * B * chunks * D) + a(4 * B * chunks * D * N) + a(4 * B * N * D) + a(4 * B * D * 8)
    assert m.mamba_selective_scan_workspace_size(1, 8192, 32, 16) == capped(1, 32, 16)
    assert m.mamba_selective_scan_workspace_size(1, 32768, 64, 16) == capped(1, 64, 16)


def test_conv_validation():
    lib = m.load_library()
    st = lib.mamba_conv1d_fwd(FAKE, 32, FAKE + (1 << 30), None, None, FAKE + (1 << 31), F32, 1, 8, 64, 4, None)
    assert st == EINVAL and "x_row_stride" in m.mamba_last_error()
    st = lib.mamba_conv1d_fwd(FAKE, 64, FAKE + (1 << 30), None, None, FAKE + (1 << 31), F32, 1, 8, 64, 9, None)
    assert st == EUNSUP and "K = 9" in m.mamba_last_error()
    st = lib.mamba_conv1d_fwd(FAKE, 64, FAKE + (1 << 30), None, None, FAKE, F32, 1, 8, 64, 4, None)
    assert st == EINVAL and "u overlaps x" in m.mamba_last_error()
    st = lib.mamba_conv1d_fwd(None, 64, None, None, None, None, F32, 1, 0, 64, 4, None)
    assert st == 0  # T == 0: nothing to do


def test_step_validation():
    lib = m.load_library()
    st = lib.mamba_conv1d_step(FAKE, 64, FAKE + (1 << 30), None, None, FAKE + (1 << 31), F32, 2, 3, 64, 4, None)
    assert st == EINVAL and "conv_state is NULL" in m.mamba_last_error()
    st = lib.mamba_conv1d_step(FAKE, 64, FAKE + (1 << 30), None, FAKE + (1 << 32), FAKE + (1 << 31), F32, 300, 300, 64, 4, None)
    assert st == EUNSUP and "L*B" in m.mamba_last_error()
    st = lib.mamba_ssm_step(FAKE, FAKE + (1 << 28), None, 1, FAKE + (1 << 29), FAKE + (1 << 30), FAKE + (1 << 31),
                            16, None, None, 0, None, FAKE + (1 << 32), F32, 2, 3, 64, 16, None)
    assert st == EINVAL and "ssm_state is NULL" in m.mamba_last_error()
    st = lib.mamba_ssm_step(FAKE, FAKE + (1 << 28), None, 1, FAKE + (1 << 29), FAKE + (1 << 30), FAKE + (1 << 31),
                            16, None, None, 0, FAKE + (1 << 33), FAKE + (1 << 32), F32, 2, 3, 64, 0, None)
    assert st == EINVAL and "N = 0" in m.mamba_last_error()
    st = lib.mamba_ssm_step(FAKE, FAKE + (1 << 28), None, 1, FAKE + (1 << 29), FAKE + (1 << 30), FAKE + (1 << 31),
                            16, None, None, 0, FAKE + (1 << 33), FAKE + (1 << 32), F32, 300, 300, 64, 16, None)
    assert st == EUNSUP and "L*B" in m.mamba_last_error()


def test_decode_step_validation():
    lib = m.load_library()
    args = lambda cs, L, B: (FAKE, 64, FAKE + (1 << 28), None, cs, FAKE + (1 << 29), None, 1, FAKE + (1 << 30),
                             FAKE + (1 << 31), FAKE + (1 << 32), 16, None, None, 0, FAKE + (1 << 33), None,
                             FAKE + (1 << 34), F32, L, B, 64, 4, 16, None)
    st = lib.mamba_decode_step(*args(None, 2, 3))
    assert st == EINVAL and "conv_state is NULL" in m.mamba_last_error()
    st = lib.mamba_decode_step(*args(FAKE + (1 << 35), 300, 300))
    assert st == EUNSUP and "L*B" in m.mamba_last_error()
    st = lib.mamba_decode_step(*args(FAKE + (1 << 33), 2, 3))
    assert st == EINVAL and "overlaps" in m.mamba_last_error()


def test_errors_are_thread_local():
    import threading
    st, msg = scan_call(u=None)
    assert st == EINVAL
    seen = {}

    def other():
        seen["msg"] = m.mamba_last_error()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["msg"] == ""
    assert "u is NULL" in m.mamba_last_error()


def m3_call(**kw):
    p = m.Mamba3SisoParams(*[FAKE + (i << 26) for i in range(1, 7)], None)
    a = dict(proj=FAKE + (1 << 33), prs=None, params=p, a_floor=1e-4, h=FAKE + (1 << 34),
             k=FAKE + (1 << 35), v=FAKE + (1 << 36), ang=FAKE + (1 << 37), out=FAKE + (1 << 38),
             L=2, B=3, nh=4, hd=8, ds=16, ng=2, na=4, stream=None)
    a.update(kw)
    if a["prs"] is None:
        a["prs"] = 2 * a["nh"] * a["hd"] + 2 * a["ng"] * a["ds"] + 3 * a["nh"] + a["na"]
    st = m.load_library().mamba3_siso_step(
        a["proj"], a["prs"], ctypes.byref(a["params"]) if a["params"] is not None else None,
        ctypes.c_float(a["a_floor"]), a["h"], a["k"], a["v"], a["ang"], a["out"], a["L"], a["B"],
        a["nh"], a["hd"], a["ds"], a["ng"], a["na"], a["stream"])
    return st, m.mamba_last_error()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(ds=18), EUNSUP, "multiple of 4"),
    (dict(ds=260), EUNSUP, "d_state = 260"),
    (dict(hd=0), EINVAL, "headdim = 0"),
    (dict(hd=300), EUNSUP, "headdim = 300"),
    (dict(ng=3), EINVAL, "not a multiple of ngroups"),
    (dict(ng=0), EINVAL, "ngroups = 0"),
    (dict(na=9), EINVAL, "n_angles = 9"),
    (dict(na=-1), EINVAL, "n_angles = -1"),
    (dict(prs=10), EINVAL, "proj_row_stride"),
    (dict(params=None), EINVAL, "params is NULL"),
    (dict(proj=None), EINVAL, "proj is NULL"),
    (dict(h=FAKE + (1 << 34) + 4), EINVAL, "ssm_state"),
    (dict(out=FAKE + (1 << 34)), EINVAL, "out overlaps ssm_state"),
    (dict(k=FAKE + (1 << 34) + 64), EINVAL, "ssm_state overlaps k_state"),
    (dict(L=-1), EINVAL, "L = -1"),
])
def test_mamba3_step_validation(kw, status, needle):
    st, msg = m3_call(**kw)
    assert st == status, msg
    assert needle in msg and msg.startswith("mamba3_siso_step"), msg


def test_mamba3_step_empty_is_noop():
    st, msg = m3_call(L=0, proj=None, h=None, k=None, v=None, ang=None, out=None)
    assert st == 0, msg


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    """The no-allocation conv + scan refuses, before any HIP call, a shape whose scan workspace
    exceeds the library's fixed 16 MiB scratch (d_state 64 over 24576 channels in 2 chunks
    needs 19857408 bytes), and says which call to use instead."""
    lib = m.load_library()
    B, T, D, K, N = 1, 176, 24576, 4, 64
    need = lib.mamba_selective_scan_workspace_size(B, T, D, N)
    assert need == 19857408 > (16 << 20)
    st = lib.mamba_conv_scan_fwd_noalloc(
        FAKE, D, FAKE, None, None, FAKE, None, 1, FAKE, FAKE, FAKE, 2 * N, None, None, 0,
        None, None, None, FAKE, F32, B, T, D, K, N, None)
    assert st == EWS
    msg = m.mamba_last_error()
    assert "mamba_conv_scan_fwd_noalloc" in msg and "19857408" in msg and str(16 << 20) in msg
    assert "mamba_conv_scan_fwd with a workspace" in msg


def test_xproj_dtproj_workspace_size():
    """x_proj's K split as the backbone prefill runs it: the 130m layer (8192 rows, d_inner
    1536, 80 output columns) takes 4 slices of 384, whose partial planes are 4 x 8192 x 80
    floats; a decode-sized M and a d_inner that is not whole 64-wide slabs take no split."""
    lib = m.load_library()
    assert lib.mamba_xproj_dtproj_workspace_size(8192, 1536, 48, 16) == 4 * 8192 * 80 * 4
    assert lib.mamba_xproj_dtproj_workspace_size(40, 1536, 48, 16) == 0
    assert lib.mamba_xproj_dtproj_workspace_size(8192, 1000, 48, 16) == 0
    assert lib.mamba_xproj_dtproj_workspace_size(-1, 1536, 48, 16) == 0


@pytest.mark.parametrize("kw,status,needle", [
    (dict(M=-1), EINVAL, "M = -1"),
    (dict(ldu=1000), EINVAL, "ldu = 1000"),
    (dict(ws=None), EWS, "workspace is NULL"),
    (dict(wsb=100), EWS, "workspace_bytes = 100"),
    (dict(xdbl=FAKE + 64), EINVAL, "xdbl overlaps u"),
    (dict(dt=FAKE + (1 << 32) + 64), EINVAL, "xdbl overlaps dt"),
    (dict(u=FAKE + 2), EINVAL, "aligned"),
])
def test_xproj_dtproj_validation(kw, status, needle):
    lib = m.load_library()
    M, D, R, N = 8192, 1536, 48, 16
    a = dict(u=FAKE, ldu=D, wx=FAKE + (1 << 30), wdt=FAKE + (1 << 31), xdbl=FAKE + (1 << 32),
             dt=FAKE + (1 << 33), M=M, ws=FAKE + (1 << 34), wsb=1 << 30)
    a.update(kw)
    st = lib.mamba_xproj_dtproj(a["u"], a["ldu"], a["wx"], a["wdt"], a["xdbl"], a["dt"], None, 0, a["M"], D, R,
                                N, a["ws"], a["wsb"], None)
    assert st == status
    assert needle in m.mamba_last_error()


def test_xproj_dtproj_empty_is_noop():
    lib = m.load_library()
    assert lib.mamba_xproj_dtproj(None, 0, None, None, None, None, None, 0, 0, 1536, 48, 16, None, 0, None) == 0


@pytest.mark.parametrize("kw,status,needle", [
    (dict(T=-1), EINVAL, "T = -1"),
    (dict(K=9), EUNSUP, "d_conv = 9"),
    (dict(xs=1000), EINVAL, "x_row_stride = 1000"),
    (dict(ws=None), EWS, "workspace is NULL"),
    (dict(u=FAKE + 64), EINVAL, "u overlaps x"),
    (dict(st=FAKE + (1 << 35) + 4), EINVAL, "dt overlaps conv_state"),
    (dict(xdbl=FAKE + (1 << 34) + 64), EINVAL, "workspace overlaps xdbl"),
    (dict(db=FAKE + (1 << 35) + 8), EINVAL, "dt overlaps dt_bias"),
    (dict(db=FAKE + (1 << 27) + 2), EINVAL, "dt_bias"),
])
def test_conv_xproj_dtproj_validation(kw, status, needle):
    lib = m.load_library()
    Bsz, T, D, R, N = 4, 2048, 1536, 48, 16
    a = dict(x=FAKE, xs=2 * D, st=FAKE + (1 << 29), u=FAKE + (1 << 30), xdbl=FAKE + (1 << 32),
             dt=FAKE + (1 << 35), db=FAKE + (1 << 27), T=T, K=4, ws=FAKE + (1 << 34), wsb=1 << 30)
    a.update(kw)
    st = lib.mamba_conv_xproj_dtproj(a["x"], a["xs"], FAKE + (1 << 28), None, a["st"], None, a["u"],
                                     FAKE + (1 << 31), FAKE + (1 << 33), a["xdbl"], a["dt"], a["db"], 1, Bsz,
                                     a["T"], D, a["K"], R, N, a["ws"], a["wsb"], None)
    assert st == status
    assert needle in m.mamba_last_error()
