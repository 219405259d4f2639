"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments with the documented status codes
before making any HIP call (so these run without a GPU).

The pointers passed here are fake, never-dereferenced addresses; every call
below fails validation, so nothing is launched.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mamba_scan.h")

from selective_state_space_75_amd import _lib  # noqa: E402

OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WS = 0, -1, -2, -3, -4, -5, -6
F32, BF16 = 0, 1


def declared_functions():
    src = open(HEADER, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mamba_[a-z0-9_]+)\s*\(", src)))


def test_header_symbols_are_exported():
    names = declared_functions()
    assert names == ["mamba_conv1d_fwd", "mamba_conv1d_update", "mamba_scan_bwd", "mamba_scan_bwd_workspace_size",
                     "mamba_scan_fwd", "mamba_scan_fwd_noalloc", "mamba_scan_kernel", "mamba_scan_workspace_size",
                     "mamba_set_test_knobs",
                     "mamba_ssd_fwd",
                     "mamba_ssd_workspace_size", "mamba_state_update", "mamba_status_string"]
    L = _lib.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for code in [OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WS, -7]:
        s = _lib.status_string(code)
        assert s and s != "unknown status"
    assert _lib.status_string(12345) == "unknown status"


def test_workspace_size_plan():
    ws = _lib.workspace_size
    assert ws(1, 16, 16, 256) == 0
    assert ws(8, 1536, 16, 2048) == 0
    # 2560 tiles of 16 channels, ten per CU: the lean row kernel, no workspace
    assert ws(8, 5120, 16, 2048) == 0
    # four or more tiles of 16 channels per CU: the lean row kernel, no workspace
    assert ws(4, 4096, 16, 2048) == 0
    # the wave-tile kernel at >= 1024 tiles of 16 channels: balanced split over
    # 1024 waves, one hand-over slot per wave (an 8-byte flag each, then 16 x 16
    # fp32 states each)
    with _lib.test_knobs(scan_kernel="wave_tile"):
        assert ws(4, 4096, 16, 2048) == 1024 * 8 + 1024 * 16 * 16 * 4
    # L % 32 != 0: the row kernel's ragged form in one pass, no hand-over; on
    # the wave-tile kernel (L % 8 == 0) the balanced split, its last chunk shifted back
    assert ws(4, 5120, 16, 2040) == 0
    assert ws(4, 5120, 16, 2044) == 0
    with _lib.test_knobs(scan_kernel="wave_tile"):
        assert ws(4, 5120, 16, 2040) == 1024 * 8 + 1024 * 16 * 16 * 4
    # the batch-1 long sequence (256 tiles): the row kernel over 4 chunks of
    # 32768 steps, its two passes with h_local and h_start (K, B, D, N) fp32
    # and the sums of delta (K, B, D) fp32 between them
    assert ws(1, 4096, 16, 131072) == 2 * 4 * 4096 * 16 * 4 + 4 * 4096 * 4
    assert ws(2, 4096, 16, 65536) == 0      # 512 tiles: the row kernel too
    with _lib.test_knobs(scan_kernel="wave_tile"):
        n = ws(1, 4096, 16, 131072)
        # 256 tiles of 16 channels -> 5 chunks (a summary pass of 4 x 256 waves,
        # a full pass of 5 x 256 (chunk, tile) pairs balanced over 1024 waves):
        # h_local and h_start (K, B, D, N) fp32, sum of delta (K, B, D) fp32, then
        # the hand-over flags and slots
        assert n == 2 * 5 * 4096 * 16 * 4 + 5 * 4096 * 4 + 1024 * 8 + 1024 * 16 * 16 * 4
        # 512 tiles -> 3 chunks; 768 tiles: one pass
        assert ws(2, 4096, 16, 65536) == 2 * 3 * 2 * 4096 * 16 * 4 + 3 * 2 * 4096 * 4 + 1024 * 8 + \
            1024 * 16 * 16 * 4
        assert ws(8, 1536, 16, 65536) == 0
    # 64 tiles: the row kernel over 13 chunks (768 / 64 + 1) of 5056 steps
    # (65536 / 13 rounded up to a multiple of 64), no hand-over area
    assert ws(1, 1024, 16, 65536) == 2 * 13 * 1024 * 16 * 4 + 13 * 1024 * 4
    # the same shape on the wave-tile kernel: 17 chunks, a balanced full pass
    with _lib.test_knobs(scan_kernel="wave_tile"):
        assert ws(1, 1024, 16, 65536) == 2 * 17 * 1024 * 16 * 4 + 17 * 1024 * 4 + 1024 * 8 + 1024 * 16 * 16 * 4
    # a ragged last chunk (L % 32 == 24 or 28): the row kernel over 4 chunks of
    # 32768 steps as at 131072 (the last one 8 or 4 steps short); on the
    # wave-tile kernel 5 chunks as above
    assert ws(1, 4096, 16, 131072 - 8) == 2 * 4 * 4096 * 16 * 4 + 4 * 4096 * 4
    assert ws(1, 4096, 16, 131072 - 4) == 2 * 4 * 4096 * 16 * 4 + 4 * 4096 * 4
    with _lib.test_knobs(scan_kernel="wave_tile"):
        assert ws(1, 4096, 16, 131072 - 8) == n
    # the general kernel plans with 64-channel tiles: 16 chunks
    with _lib.test_knobs(scan_kernel="general"):
        assert ws(1, 4096, 16, 131072 - 4) == 2 * 16 * 4096 * 16 * 4 + 16 * 4096 * 4
    assert _lib.lib().mamba_scan_workspace_size(0, 1, 1, 1) == ctypes.c_size_t(-1).value
    assert _lib.lib().mamba_scan_workspace_size(1, 1, 17, 1) == ctypes.c_size_t(-1).value


def test_forced_chunks_knob():
    # 5 forced chunks x 256 tiles: summary workspace plus the hand-over area
    with _lib.test_knobs(scan_chunks=5):
        assert _lib.workspace_size(1, 4096, 16, 320) == 2 * 5 * 4096 * 16 * 4 + 5 * 4096 * 4 + 1024 * 8 + \
            1024 * 16 * 16 * 4
    with _lib.test_knobs(scan_chunks=3):
        # L = 100 -> chunk_len rounds 34 up to 64 -> 2 chunks
        assert _lib.workspace_size(2, 70, 5, 100) == 2 * (((2 * 2 * 70 * 5 * 4) + 255) // 256 * 256) + \
            ((2 * 2 * 70 * 4 + 255) // 256 * 256)
    with _lib.test_knobs(scan_chunks=1):
        assert _lib.workspace_size(2, 70, 5, 100) == 0
    # back to the planner: one pass, no workspace
    assert _lib.workspace_size(2, 70, 5, 100) == 0
    assert _lib.workspace_size(1, 4096, 16, 320) == 0


def test_knob_defaults_and_errors():
    import pytest as _pt
    # on the wave-tile kernel, no balance drops the hand-over area
    with _lib.test_knobs(scan_kernel="wave_tile", scan_no_balance=True):
        assert _lib.workspace_size(4, 4096, 16, 2048) == 0
    with _lib.test_knobs(scan_kernel="wave_tile"):
        assert _lib.workspace_size(4, 4096, 16, 2048) == 1024 * 8 + 1024 * 16 * 16 * 4
    with _pt.raises(_lib.MambaError):
        _lib.set_test_knobs(scan_chunks=-1)
    with _lib.test_knobs(ssd_segments=3):
        assert _lib.ssd_workspace_size(4, 80, 64, 128, 2048) > 0
    assert _lib.lib().mamba_set_test_knobs(None) == 0


P = 0x10000  # fake 64 KiB-aligned device address, never dereferenced


def scan(**kw):
    a = dict(u=P, delta=P, z=P, Bt=P, Ct=P, A=P, Dskip=P, bias=P, y=P, fs=P, B=2, D=64, N=16, L=64,
             ind=BF16, outd=BF16, rfs=1, flags=0, ws=None, wsb=0)
    a.update(kw)
    vp = lambda v: ctypes.c_void_p(v) if v is not None else None  # noqa: E731
    return _lib.lib().mamba_scan_fwd(vp(a["u"]), vp(a["delta"]), vp(a["z"]), vp(a["Bt"]), vp(a["Ct"]),
                                     vp(a["A"]), vp(a["Dskip"]), vp(a["bias"]), vp(a["y"]), vp(a["fs"]),
                                     a["B"], a["D"], a["N"], a["L"], a["ind"], a["outd"], a["rfs"],
                                     a["flags"], vp(a["ws"]), a["wsb"], None)


def update(**kw):
    a = dict(st=P, u=P, delta=P, z=P, Bt=P, Ct=P, A=P, Dskip=P, bias=P, y=P, B=2, D=64, N=16,
             ind=BF16, outd=BF16, flags=0)
    a.update(kw)
    vp = lambda v: ctypes.c_void_p(v) if v is not None else None  # noqa: E731
    return _lib.lib().mamba_state_update(vp(a["st"]), vp(a["u"]), vp(a["delta"]), vp(a["z"]), vp(a["Bt"]),
                                         vp(a["Ct"]), vp(a["A"]), vp(a["Dskip"]), vp(a["bias"]), vp(a["y"]),
                                         a["B"], a["D"], a["N"], a["ind"], a["outd"], a["flags"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(ind=7), DTYPE), (dict(outd=-1), DTYPE),
    (dict(flags=0x100), UNSUP),
    (dict(B=0), SHAPE), (dict(D=-3), SHAPE), (dict(L=0), SHAPE), (dict(N=0), SHAPE),
    (dict(B=1 << 20, D=1 << 20, L=1 << 20), SHAPE),
    (dict(N=17), UNSUP),
    (dict(u=None), NULL), (dict(delta=None), NULL), (dict(Bt=None), NULL), (dict(Ct=None), NULL),
    (dict(A=None), NULL), (dict(y=None), NULL), (dict(fs=None), NULL),
    (dict(u=P + 2), ALIGN), (dict(z=P + 8), ALIGN), (dict(y=P + 4), ALIGN), (dict(Ct=P + 2), ALIGN),
    (dict(A=P + 2), ALIGN), (dict(fs=P + 1), ALIGN),
    # the row kernel over chunks needs a workspace (the carried states of the
    # batch-1 long sequence, aligned or ragged)
    (dict(B=1, D=4096, L=131072), WS),
    (dict(B=1, D=4096, L=131072, ws=P, wsb=1024), WS),
    (dict(B=1, D=4096, L=131064), WS),
])
def test_scan_rejects_bad_arguments(kw, code):
    assert scan(**kw) == code


def test_scan_optional_pointers_do_not_trigger_errors_early():
    # z, Dskip, bias may be NULL and final state is ignored when not requested;
    # with everything else valid but the workspace missing, the workspace error
    # is what comes back (so no launch happens).
    st = scan(z=None, Dskip=None, bias=None, fs=None, rfs=0, B=1, D=4096, L=131072)
    assert st == WS


@pytest.mark.parametrize("kw,code", [
    (dict(ind=2), DTYPE), (dict(flags=0x8), UNSUP), (dict(B=0), SHAPE), (dict(N=17), UNSUP),
    (dict(st=None), NULL), (dict(u=None), NULL), (dict(Bt=None), NULL), (dict(A=None), NULL),
    (dict(y=None), NULL), (dict(st=P + 4), ALIGN), (dict(A=P + 8), ALIGN), (dict(u=P + 1), ALIGN),
    (dict(ind=F32, u=P + 2), ALIGN), (dict(Dskip=P + 2), ALIGN), (dict(outd=F32, y=P + 2), ALIGN),
])
def test_update_rejects_bad_arguments(kw, code):
    assert update(**kw) == code


def test_python_binding_rejects_before_calling():
    torch = pytest.importorskip("torch")
    import selective_state_space_75_amd as m
    x = torch.zeros(1, 2, 8)
    with pytest.raises(ValueError):
        m.scan_fwd(x, x, x, torch.zeros(1, 3, 8), torch.zeros(1, 3, 8), torch.zeros(2, 3))


def conv(**kw):
    a = dict(x=P, w=P, bias=P, y=P, fs=P, B=2, D=64, L=64, K=4, ind=BF16, outd=BF16, rfs=1)
    a.update(kw)
    vp = lambda v: ctypes.c_void_p(v) if v is not None else None  # noqa: E731
    return _lib.lib().mamba_conv1d_fwd(vp(a["x"]), vp(a["w"]), vp(a["bias"]), vp(a["y"]), vp(a["fs"]),
                                       a["B"], a["D"], a["L"], a["K"], a["ind"], a["outd"], a["rfs"], None)


def conv_update(**kw):
    a = dict(st=P, x=P, w=P, bias=P, y=P, B=2, D=64, K=4, ind=BF16, outd=BF16)
    a.update(kw)
    vp = lambda v: ctypes.c_void_p(v) if v is not None else None  # noqa: E731
    return _lib.lib().mamba_conv1d_update(vp(a["st"]), vp(a["x"]), vp(a["w"]), vp(a["bias"]), vp(a["y"]),
                                          a["B"], a["D"], a["K"], a["ind"], a["outd"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(ind=5), DTYPE), (dict(outd=9), DTYPE),
    (dict(B=0), SHAPE), (dict(L=-1), SHAPE), (dict(K=0), SHAPE), (dict(K=5), UNSUP),
    (dict(B=1 << 20, D=1 << 20, L=1 << 20), SHAPE),
    (dict(x=None), NULL), (dict(w=None), NULL), (dict(y=None), NULL), (dict(fs=None), NULL),
    (dict(x=P + 1), ALIGN), (dict(ind=F32, x=P + 2), ALIGN), (dict(outd=F32, y=P + 2), ALIGN),
    (dict(w=P + 2), ALIGN), (dict(bias=P + 1), ALIGN), (dict(fs=P + 2), ALIGN),
])
def test_conv_rejects_bad_arguments(kw, code):
    assert conv(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(ind=3), DTYPE), (dict(B=0), SHAPE), (dict(K=0), SHAPE), (dict(K=7), UNSUP),
    (dict(st=None), NULL), (dict(x=None), NULL), (dict(w=None), NULL), (dict(y=None), NULL),
    (dict(st=P + 2), ALIGN), (dict(x=P + 1), ALIGN), (dict(w=P + 1), ALIGN),
])
def test_conv_update_rejects_bad_arguments(kw, code):
    assert conv_update(**kw) == code


def test_conv_optional_pointers():
    # bias may be NULL and final_state is ignored when not requested: with every
    # other argument valid the call only fails at the size check we force here
    assert conv(bias=None, fs=None, rfs=0, K=9) == UNSUP


def test_bwd_workspace_size():
    ws = _lib.scan_bwd_workspace_size
    a = lambda x: (x + 255) // 256 * 256  # noqa: E731
    B, D, N, L = 2, 70, 5, 100
    # 5 channel tiles in 2 workgroups of up to 4; one stored state per
    # 32-step block -> 4 blocks; segments: 10 (row, tile) pairs want 820
    # segments, at most ceil(100 / 64) = 2 -> 50 steps, rounded up to 64 -> 2
    groups, nck, S = 2, 4, 2
    bd, bsd = B * D, B * D * S
    assert ws(B, D, N, L) == (a(bd * nck * 16 * 4) + a(bd * nck * 4) + 5 * a(bsd * 16 * 4)
                              + 2 * a(B * groups * 16 * L * 4) + a(bsd * 16 * 4) + 2 * a(bsd * 4))
    assert _lib.lib().mamba_scan_bwd_workspace_size(1, 1, 17, 1) == ctypes.c_size_t(-1).value


def bwd(**kw):
    a = dict(u=P, delta=P, z=P, Bt=P, Ct=P, A=P, Dskip=P, bias=P, dy=P, du=P, ddelta=P, dz=P, dBt=P, dCt=P,
             dA=P, dD=P, dbias=P, B=2, D=64, N=16, L=64, ind=BF16, gd=F32, flags=0, ws=P, wsb=1 << 40)
    a.update(kw)
    vp = lambda v: ctypes.c_void_p(v) if v is not None else None  # noqa: E731
    return _lib.lib().mamba_scan_bwd(*[vp(a[k]) for k in ("u", "delta", "z", "Bt", "Ct", "A", "Dskip", "bias", "dy",
                                                         "du", "ddelta", "dz", "dBt", "dCt", "dA", "dD", "dbias")],
                                     a["B"], a["D"], a["N"], a["L"], a["ind"], a["gd"], a["flags"], vp(a["ws"]),
                                     a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(ind=4), DTYPE), (dict(gd=-2), DTYPE), (dict(flags=0x40), UNSUP),
    (dict(B=0), SHAPE), (dict(N=17), UNSUP),
    (dict(u=None), NULL), (dict(dy=None), NULL), (dict(dBt=None), NULL), (dict(dA=None), NULL),
    (dict(dz=None), NULL), (dict(dbias=None), NULL),
    (dict(u=P + 1), ALIGN), (dict(dy=P + 2), ALIGN), (dict(dA=P + 2), ALIGN),
    (dict(ws=None), WS), (dict(wsb=1024), WS), (dict(ws=P + 16), ALIGN),
])
def test_bwd_rejects_bad_arguments(kw, code):
    assert bwd(**kw) == code


def ssd(**kw):
    a = dict(x=P, delta=P, z=P, Bt=P, Ct=P, A=P, Dskip=P, bias=P, y=P, fs=P, B=2, H=4, Pd=64, N=128, L=64,
             ind=BF16, outd=BF16, rfs=1, flags=0, ws=None, wsb=0)
    a.update(kw)
    vp = lambda v: ctypes.c_void_p(v) if v is not None else None  # noqa: E731
    return _lib.lib().mamba_ssd_fwd(vp(a["x"]), vp(a["delta"]), vp(a["z"]), vp(a["Bt"]), vp(a["Ct"]), vp(a["A"]),
                                    vp(a["Dskip"]), vp(a["bias"]), vp(a["y"]), vp(a["fs"]), a["B"], a["H"], a["Pd"],
                                    a["N"], a["L"], a["ind"], a["outd"], a["rfs"], a["flags"], vp(a["ws"]), a["wsb"],
                                    None)


@pytest.mark.parametrize("kw,code", [
    (dict(ind=4), DTYPE), (dict(outd=3), DTYPE), (dict(flags=0x2), UNSUP), (dict(flags=0x10), UNSUP),
    (dict(B=0), SHAPE), (dict(H=0), SHAPE), (dict(Pd=0), SHAPE), (dict(L=0), SHAPE), (dict(N=0), SHAPE),
    (dict(B=1 << 20, H=1 << 20, L=1 << 20), SHAPE),
    (dict(ind=F32), UNSUP), (dict(N=16), UNSUP), (dict(N=96), UNSUP), (dict(Pd=32), UNSUP), (dict(Pd=96), UNSUP),
    (dict(x=None), NULL), (dict(delta=None), NULL), (dict(Bt=None), NULL), (dict(Ct=None), NULL),
    (dict(A=None), NULL), (dict(y=None), NULL), (dict(fs=None), NULL),
    (dict(x=P + 1), ALIGN), (dict(Ct=P + 1), ALIGN), (dict(outd=F32, y=P + 2), ALIGN), (dict(A=P + 2), ALIGN),
    (dict(fs=P + 2), ALIGN), (dict(Dskip=P + 1), ALIGN),
    # long enough to be cut into segments: a workspace is needed
    (dict(B=1, H=2, L=4096), WS), (dict(B=1, H=2, L=4096, ws=P, wsb=64), WS),
    (dict(B=1, H=2, L=4096, ws=P + 16, wsb=1 << 40), ALIGN),
])
def test_ssd_rejects_bad_arguments(kw, code):
    assert ssd(**kw) == code


def test_ssd_workspace_size():
    ws = _lib.ssd_workspace_size
    a = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert ws(1, 2, 64, 128, 200) == 0                    # one segment (L < 2 x 256)
    # B=4, 80 heads of one 64-channel block: 320 workgroups want 4 segments
    # (about 1024 workgroups) of 512 steps: one state slot per workgroup
    slots = 4 * 320
    assert ws(4, 80, 64, 128, 2048) == a(slots * 64 * 128 * 4) + a(slots * 4)
    # 512 workgroups or more: one segment
    assert ws(8, 64, 64, 128, 2048) == 0
    # B=1, 8 heads: 8 workgroups want 128 segments of 512 steps
    slots = 128 * 8
    assert ws(1, 8, 64, 128, 65536) == a(slots * 64 * 128 * 4) + a(slots * 4)
    # 1 x 2 blocks want 128 segments; at most ceil(1000 / 256) = 4 -> 250 -> 256 steps -> 4
    assert ws(1, 2, 64, 64, 1000) == a(1 * 4 * 2 * 64 * 64 * 4) + a(1 * 4 * 2 * 4)
    assert _lib.lib().mamba_ssd_workspace_size(1, 2, 64, 16, 100) == ctypes.c_size_t(-1).value


def test_noalloc_refuses_oversized_plan():
    """mamba_scan_fwd_noalloc's scratch buffer holds 8 MiB.  The planner's own
    plans stay far below it (the batch-1 long sequence needs 3.75 MiB); 64
    forced chunks over 16384 channels need 134 MB of carries, so the call is
    refused in its host checks, before any HIP call (the fake pointers are
    never dereferenced)."""
    from selective_state_space_75_amd import workloads as W
    B, D, N, L = 1, 16384, 16, 1 << 16
    with _lib.test_knobs(scan_chunks=64):
        assert _lib.workspace_size(B, D, N, L) > (8 << 20)
        st = scan_noalloc(B=B, D=D, N=N, L=L)
    assert st == WS, "expected MAMBA_ERR_WORKSPACE, got %d" % st
    cfg = W.SCAN_CONFIGS["long_b1"]
    assert _lib.workspace_size(cfg.B, cfg.D, cfg.N, cfg.L) <= (8 << 20)
    # argument checks come first, as in mamba_scan_fwd
    assert scan_noalloc(N=17) == UNSUP
    assert scan_noalloc(u=None) == NULL
    assert scan_noalloc(u=P + 2) == ALIGN


def scan_noalloc(**kw):
    a = dict(u=P, delta=P, z=P, Bt=P, Ct=P, A=P, Dskip=P, bias=P, y=P, fs=P, B=2, D=64, N=16, L=64,
             ind=BF16, outd=BF16, rfs=1, flags=0)
    a.update(kw)
    vp = lambda v: ctypes.c_void_p(v) if v is not None else None  # noqa: E731
    return _lib.lib().mamba_scan_fwd_noalloc(vp(a["u"]), vp(a["delta"]), vp(a["z"]), vp(a["Bt"]), vp(a["Ct"]),
                                             vp(a["A"]), vp(a["Dskip"]), vp(a["bias"]), vp(a["y"]), vp(a["fs"]),
                                             a["B"], a["D"], a["N"], a["L"], a["ind"], a["outd"], a["rfs"],
                                             a["flags"], None)


def test_scan_kernel_choice():
    """The planner's kernel per workload: the lean row kernel from four
    16-channel workgroups per CU on (the 2.8B layer has five) when L % 32 ==
    0, the row kernel where 16-channel wave tiles would leave SIMDs idle or
    need chunking (130M layer, batch-1 long sequence) and, by its cost model,
    at L % 32 != 0 (its ragged form), chunking of the wave-tile kernel for
    very few tiles over long L when L % 8 == 0, the general kernel only below
    32 steps.  (Each choice was the fastest kernel in an interleaved timing
    of all of them on MI355X.)"""
    k = _lib.scan_kernel
    assert k(8, 1536, 16, 2048) == "row"       # 768 tiles: 3 per CU
    assert k(1, 4096, 16, 131072) == "row"     # in 4 chunks
    assert k(4, 5120, 16, 2048) == "row_lean"
    assert k(5, 4096, 16, 2048) == "row_lean"
    assert k(7, 4096, 16, 2048) == "row_lean"
    assert k(4, 4096, 16, 2048) == "row_lean"
    assert k(3, 5120, 16, 2048) == "row_lean"  # 960 tiles: 3.75 per CU, rounded up to 4
    assert k(3, 4096, 16, 2048) == "row"       # 768 tiles: 3 per CU
    assert k(2, 4096, 16, 2048) == "row"       # 512 tiles: 2 per CU
    assert k(4, 3584, 16, 2048) == "row_lean"  # 896 tiles: 3.5 per CU, rounded up to 4
    assert k(4, 5120, 16, 2040) == "row"       # the lean kernel has no ragged form
    assert k(8, 1536, 16, 2040) == "row"
    assert k(1, 4096, 16, 131072 - 8) == "row"   # in 4 chunks
    assert k(1, 256, 16, 65536 - 8) == "wave_tile"   # 16 tiles: the wave-tile kernel's chunks
    assert k(1, 1024, 16, 65536) == "row"     # 13 chunks
    assert k(1, 2048, 16, 16384) == "row"     # 7 chunks (L / 2048 caps 768 / 128 + 1)
    assert k(1, 5120, 16, 8192) == "row"      # 3 chunks
    assert k(1, 256, 16, 65536) == "wave_tile"
    assert k(2, 2560, 16, 4096) == "row"
    assert k(8, 5120, 16, 2048) == "row_lean"
    assert k(32, 1536, 16, 2048) == "row_lean"
    assert k(9, 4096, 16, 2048) == "row_lean"
    assert k(2, 100, 16, 100) == "row"
    assert k(4, 5120, 16, 2044) == "row"
    assert k(1, 4096, 16, 131072 - 4) == "row"
    assert k(1, 16, 16, 33) == "row"
    assert k(1, 16, 16, 31) == "general"
    assert k(1, 16, 16, 16) == "general"
    with _lib.test_knobs(scan_kernel="wave_tile"):
        assert k(8, 1536, 16, 2048) == "wave_tile"
    with _lib.test_knobs(scan_kernel="row"):
        assert k(4, 5120, 16, 2048) == "row"
        assert k(4, 5120, 16, 2040) == "row"          # forced: any L >= 32
        assert k(4, 5120, 16, 16) == "general"
    with _lib.test_knobs(scan_kernel="row_lean"):
        assert k(8, 1536, 16, 2048) == "row_lean"
        assert k(4, 5120, 16, 2040) == "row"          # the lean variant needs L % 32 == 0
        # it counts chunks in 32 bits: L < 2^33 only (the planner's own choice
        # of it implies L < 2^32, since it needs B D >= 12,304)
        assert k(1, 16, 16, (1 << 33) - 32) == "row_lean"
        assert k(1, 16, 16, 1 << 33) == "row"
    with _lib.test_knobs(scan_kernel="general"):
        assert k(4, 5120, 16, 2048) == "general"
    assert _lib.lib().mamba_scan_kernel(1, 1, 17, 1) == UNSUP
    assert _lib.lib().mamba_scan_kernel(0, 1, 1, 1) == SHAPE
