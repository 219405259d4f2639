"""ctypes binding of libmamba_scan.so (the C ABI of include/mamba_scan.h).

Argument marshalling only: tensors are checked (device, dtype, shape,
contiguity), outputs and the workspace are allocated with torch, and raw
device pointers plus torch's current HIP stream are handed to the library.
Every step of the computation runs in the library's HIP kernels; there is no
fallback.  If the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmamba_scan.so")

MAMBA_F32, MAMBA_BF16 = 0, 1
FLAG_DELTA_B = 0x1
FLAG_ACCURATE_EXPM1 = 0x2

STATUS = {
    0: "MAMBA_OK", -1: "MAMBA_ERR_NULL", -2: "MAMBA_ERR_SHAPE", -3: "MAMBA_ERR_DTYPE",
    -4: "MAMBA_ERR_ALIGN", -5: "MAMBA_ERR_UNSUPPORTED", -6: "MAMBA_ERR_WORKSPACE", -7: "MAMBA_ERR_HIP",
}

_lock = threading.Lock()
_lib = None


class TestKnobs(ctypes.Structure):
    """mamba_test_knobs_t of include/mamba_scan.h."""
    _fields_ = [("scan_chunks", ctypes.c_int64), ("scan_kernel", ctypes.c_int32),
                ("scan_no_balance", ctypes.c_int32), ("handover_spin", ctypes.c_int64),
                ("ssd_segments", ctypes.c_int64)]


class MambaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (what, STATUS.get(status, status), status_string(status)))


def lib() -> ctypes.CDLL:
    """The loaded library with argument types set.  Raises if it is not built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libmamba_scan.so is not built (%s); run "
                                   "`python -m selective_state_space_75_amd.build`" % LIB_PATH)
            L = ctypes.CDLL(LIB_PATH)
            vp, i64, u32, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint, ctypes.c_int
            L.mamba_scan_workspace_size.argtypes = [i64, i64, i64, i64]
            L.mamba_scan_workspace_size.restype = ctypes.c_size_t
            L.mamba_scan_fwd.argtypes = ([vp] * 10 + [i64] * 4 + [c_int, c_int, c_int, u32, vp,
                                                                 ctypes.c_size_t, vp])
            L.mamba_scan_fwd.restype = c_int
            L.mamba_scan_fwd_noalloc.argtypes = [vp] * 10 + [i64] * 4 + [c_int, c_int, c_int, u32, vp]
            L.mamba_scan_fwd_noalloc.restype = c_int
            L.mamba_state_update.argtypes = [vp] * 10 + [i64] * 3 + [c_int, c_int, u32, vp]
            L.mamba_state_update.restype = c_int
            L.mamba_scan_bwd_workspace_size.argtypes = [i64, i64, i64, i64]
            L.mamba_scan_bwd_workspace_size.restype = ctypes.c_size_t
            L.mamba_scan_bwd.argtypes = [vp] * 17 + [i64] * 4 + [c_int, c_int, u32, vp, ctypes.c_size_t, vp]
            L.mamba_scan_bwd.restype = c_int
            L.mamba_conv1d_fwd.argtypes = [vp] * 5 + [i64] * 4 + [c_int, c_int, c_int, vp]
            L.mamba_conv1d_fwd.restype = c_int
            L.mamba_conv1d_update.argtypes = [vp] * 5 + [i64] * 3 + [c_int, c_int, vp]
            L.mamba_conv1d_update.restype = c_int
            L.mamba_ssd_fwd.argtypes = [vp] * 10 + [i64] * 5 + [c_int, c_int, c_int, u32, vp, ctypes.c_size_t, vp]
            L.mamba_ssd_fwd.restype = c_int
            L.mamba_ssd_workspace_size.argtypes = [i64] * 5
            L.mamba_ssd_workspace_size.restype = ctypes.c_size_t
            L.mamba_scan_kernel.argtypes = [i64, i64, i64, i64]
            L.mamba_scan_kernel.restype = c_int
            L.mamba_set_test_knobs.argtypes = [ctypes.POINTER(TestKnobs)]
            L.mamba_set_test_knobs.restype = c_int
            L.mamba_status_string.argtypes = [c_int]
            L.mamba_status_string.restype = ctypes.c_char_p
            _lib = L
    return _lib


def status_string(status: int) -> str:
    try:
        return lib().mamba_status_string(int(status)).decode()
    except Exception:
        return "?"


SCAN_KERNELS = {"planner": 0, "general": 1, "wave_tile": 2, "row": 3, "row_lean": 4}


def set_test_knobs(scan_chunks: int = 0, scan_kernel: str = "planner", scan_no_balance: bool = False,
                   handover_spin: int = -1, ssd_segments: int = 0) -> None:
    """Process-wide test knobs of the library (mamba_set_test_knobs); no
    arguments restores the defaults.  scan_kernel: planner, general,
    wave_tile, row or row_lean."""
    k = TestKnobs(scan_chunks, SCAN_KERNELS[scan_kernel], int(scan_no_balance), handover_spin, ssd_segments)
    st = lib().mamba_set_test_knobs(ctypes.byref(k))
    if st != 0:
        raise MambaError(st, "mamba_set_test_knobs")


class test_knobs:  # noqa: N801 (used as a context manager)
    """``with test_knobs(scan_chunks=5): ...`` sets the knobs for the block and
    restores the defaults after it."""
    __test__ = False   # not a pytest test class

    def __init__(self, **kw):
        self.kw = kw

    def __enter__(self):
        set_test_knobs(**self.kw)
        return self

    def __exit__(self, *exc):
        set_test_knobs()
        return False


def scan_kernel(B: int, D: int, N: int, L: int) -> str:
    """Name of the kernel mamba_scan_fwd runs for this shape (mamba_scan_kernel)."""
    k = lib().mamba_scan_kernel(B, D, N, L)
    if k < 0:
        raise MambaError(k, "mamba_scan_kernel")
    return {1: "general", 2: "wave_tile", 3: "row", 4: "row_lean"}[k]


def workspace_size(B: int, D: int, N: int, L: int) -> int:
    n = lib().mamba_scan_workspace_size(B, D, N, L)
    if n == ctypes.c_size_t(-1).value:
        raise MambaError(-2, "mamba_scan_workspace_size")
    return n


# ----------------------------------------------------------------------------- torch marshalling
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return MAMBA_BF16
    if t.dtype == torch.float32:
        return MAMBA_F32
    raise TypeError("unsupported dtype %s (bfloat16 or float32)" % t.dtype)


def _check(t, name, shape, dtype, device):
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def scan_fwd(u, delta, z, Bt, Ct, A, Dskip=None, delta_bias=None, *, return_final_state=False,
             out_dtype=None, delta_b=False, accurate_expm1=False, y=None, final_state=None,
             workspace=None, stream=None):
    """Selective scan forward.  u, delta, z: (B, D, L); Bt, Ct: (B, N, L); A: (D, N) fp32.

    Returns y (B, D, L), or (y, final_state (B, D, N) fp32) when return_final_state.
    Outputs and workspace may be passed in to avoid allocation.
    """
    torch = _torch()
    if u.dim() != 3 or Bt.dim() != 3:
        raise ValueError("u must be (B, D, L) and Bt (B, N, L)")
    B, D, L = u.shape
    N = Bt.shape[1]
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    in_dt = u.dtype
    _dtype_code(u)
    _check(u, "u", (B, D, L), in_dt, dev)
    _check(delta, "delta", (B, D, L), in_dt, dev)
    _check(z, "z", (B, D, L), in_dt, dev)
    _check(Bt, "Bt", (B, N, L), in_dt, dev)
    _check(Ct, "Ct", (B, N, L), in_dt, dev)
    _check(A, "A", (D, N), torch.float32, dev)
    _check(Dskip, "Dskip", (D,), torch.float32, dev)
    _check(delta_bias, "delta_bias", (D,), torch.float32, dev)
    out_dt = in_dt if out_dtype is None else out_dtype
    if y is None:
        y = torch.empty((B, D, L), dtype=out_dt, device=dev)
    _check(y, "y", (B, D, L), out_dt, dev)
    if return_final_state:
        if final_state is None:
            final_state = torch.empty((B, D, N), dtype=torch.float32, device=dev)
        _check(final_state, "final_state", (B, D, N), torch.float32, dev)
    ws_bytes = workspace_size(B, D, N, L)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    flags = (FLAG_DELTA_B if delta_b else 0) | (FLAG_ACCURATE_EXPM1 if accurate_expm1 else 0)
    st = lib().mamba_scan_fwd(
        _ptr(u), _ptr(delta), _ptr(z), _ptr(Bt), _ptr(Ct), _ptr(A), _ptr(Dskip), _ptr(delta_bias),
        _ptr(y), _ptr(final_state if return_final_state else None), B, D, N, L,
        _dtype_code(u), _dtype_code(y), 1 if return_final_state else 0, flags,
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(dev, stream))
    if st != 0:
        raise MambaError(st, "mamba_scan_fwd")
    return (y, final_state) if return_final_state else y


def scan_fwd_noalloc(u, delta, z, Bt, Ct, A, Dskip=None, delta_bias=None, *, y, final_state=None,
                     out_dtype=None, delta_b=False, accurate_expm1=False, stream=None):
    """scan_fwd through mamba_scan_fwd_noalloc: the library's own per-GPU
    scratch instead of a workspace, and caller-provided outputs (y, and
    final_state when given), so nothing is allocated."""
    B, D, L = u.shape
    N = Bt.shape[1]
    dev = u.device
    in_dt = u.dtype
    _dtype_code(u)
    for t, name, shape, dt in ((u, "u", (B, D, L), in_dt), (delta, "delta", (B, D, L), in_dt),
                               (z, "z", (B, D, L), in_dt), (Bt, "Bt", (B, N, L), in_dt),
                               (Ct, "Ct", (B, N, L), in_dt), (A, "A", (D, N), _torch().float32),
                               (Dskip, "Dskip", (D,), _torch().float32),
                               (delta_bias, "delta_bias", (D,), _torch().float32)):
        _check(t, name, shape, dt, dev)
    _check(y, "y", (B, D, L), y.dtype if out_dtype is None else out_dtype, dev)
    _check(final_state, "final_state", (B, D, N), _torch().float32, dev)
    flags = (FLAG_DELTA_B if delta_b else 0) | (FLAG_ACCURATE_EXPM1 if accurate_expm1 else 0)
    st = lib().mamba_scan_fwd_noalloc(
        _ptr(u), _ptr(delta), _ptr(z), _ptr(Bt), _ptr(Ct), _ptr(A), _ptr(Dskip), _ptr(delta_bias),
        _ptr(y), _ptr(final_state), B, D, N, L, _dtype_code(u), _dtype_code(y),
        1 if final_state is not None else 0, flags, _stream(dev, stream))
    if st != 0:
        raise MambaError(st, "mamba_scan_fwd_noalloc")
    return (y, final_state) if final_state is not None else y


def ssd_workspace_size(B: int, H: int, P: int, N: int, L: int) -> int:
    n = lib().mamba_ssd_workspace_size(B, H, P, N, L)
    if n == ctypes.c_size_t(-1).value:
        raise MambaError(-5, "mamba_ssd_workspace_size")
    return n


def ssd_fwd(x, delta, z, Bt, Ct, A, Dskip=None, delta_bias=None, *, P=64, return_final_state=False,
            out_dtype=None, delta_b=False, y=None, final_state=None, workspace=None, stream=None):
    """Mamba-2 (SSD) layer forward.  x, z: (B, H*P, L) bf16; delta: (B, H, L) bf16;
    Bt, Ct: (B, N, L) bf16; A, delta_bias: (H) fp32; Dskip: (H*P) fp32.

    Returns y (B, H*P, L), or (y, final_state (B, H*P, N) fp32) when return_final_state.
    """
    torch = _torch()
    if x.dim() != 3 or Bt.dim() != 3 or delta.dim() != 3:
        raise ValueError("x must be (B, H*P, L), delta (B, H, L) and Bt (B, N, L)")
    B, D, L = x.shape
    H = delta.shape[1]
    N = Bt.shape[1]
    if H * P != D:
        raise ValueError("x has %d channels, delta %d heads of P = %d" % (D, H, P))
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    in_dt = x.dtype
    _dtype_code(x)
    _check(x, "x", (B, D, L), in_dt, dev)
    _check(delta, "delta", (B, H, L), in_dt, dev)
    _check(z, "z", (B, D, L), in_dt, dev)
    _check(Bt, "Bt", (B, N, L), in_dt, dev)
    _check(Ct, "Ct", (B, N, L), in_dt, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(Dskip, "Dskip", (D,), torch.float32, dev)
    _check(delta_bias, "delta_bias", (H,), torch.float32, dev)
    out_dt = in_dt if out_dtype is None else out_dtype
    if y is None:
        y = torch.empty((B, D, L), dtype=out_dt, device=dev)
    _check(y, "y", (B, D, L), out_dt, dev)
    if return_final_state:
        if final_state is None:
            final_state = torch.empty((B, D, N), dtype=torch.float32, device=dev)
        _check(final_state, "final_state", (B, D, N), torch.float32, dev)
    ws_bytes = ssd_workspace_size(B, H, P, N, L) if (N in (64, 128) and P % 64 == 0) else 0
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    st = lib().mamba_ssd_fwd(
        _ptr(x), _ptr(delta), _ptr(z), _ptr(Bt), _ptr(Ct), _ptr(A), _ptr(Dskip), _ptr(delta_bias),
        _ptr(y), _ptr(final_state if return_final_state else None), B, H, P, N, L,
        _dtype_code(x), _dtype_code(y), 1 if return_final_state else 0, FLAG_DELTA_B if delta_b else 0,
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(dev, stream))
    if st != 0:
        raise MambaError(st, "mamba_ssd_fwd")
    return (y, final_state) if return_final_state else y


def state_update(state, u, delta, z, Bt, Ct, A, Dskip=None, delta_bias=None, *, out_dtype=None,
                 delta_b=False, accurate_expm1=False, y=None, stream=None):
    """One decoding step; `state` (B, D, N) fp32 is updated in place.  Returns y (B, D)."""
    torch = _torch()
    if state.dim() != 3:
        raise ValueError("state must be (B, D, N)")
    B, D, N = state.shape
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    in_dt = u.dtype
    _dtype_code(u)
    _check(state, "state", (B, D, N), torch.float32, dev)
    _check(u, "u", (B, D), in_dt, dev)
    _check(delta, "delta", (B, D), in_dt, dev)
    _check(z, "z", (B, D), in_dt, dev)
    _check(Bt, "Bt", (B, N), in_dt, dev)
    _check(Ct, "Ct", (B, N), in_dt, dev)
    _check(A, "A", (D, N), torch.float32, dev)
    _check(Dskip, "Dskip", (D,), torch.float32, dev)
    _check(delta_bias, "delta_bias", (D,), torch.float32, dev)
    out_dt = in_dt if out_dtype is None else out_dtype
    if y is None:
        y = torch.empty((B, D), dtype=out_dt, device=dev)
    _check(y, "y", (B, D), out_dt, dev)
    st = lib().mamba_state_update(
        _ptr(state), _ptr(u), _ptr(delta), _ptr(z), _ptr(Bt), _ptr(Ct), _ptr(A), _ptr(Dskip),
        _ptr(delta_bias), _ptr(y), B, D, N, _dtype_code(u), _dtype_code(y),
        (FLAG_DELTA_B if delta_b else 0) | (FLAG_ACCURATE_EXPM1 if accurate_expm1 else 0),
        _stream(dev, stream))
    if st != 0:
        raise MambaError(st, "mamba_state_update")
    return y


def conv1d_fwd(x, weight, bias=None, *, return_final_state=False, out_dtype=None, y=None, final_state=None,
               stream=None):
    """Causal depthwise conv1d + SiLU.  x: (B, D, L); weight: (D, K) fp32 with
    weight[d, i] multiplying x[..., t - i]; bias: (D) fp32 or None.

    Returns y (B, D, L), or (y, final_state (B, D, K) fp32) when return_final_state.
    """
    torch = _torch()
    if x.dim() != 3 or weight.dim() != 2:
        raise ValueError("x must be (B, D, L) and weight (D, K)")
    B, D, L = x.shape
    K = weight.shape[1]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    _dtype_code(x)
    _check(x, "x", (B, D, L), x.dtype, dev)
    _check(weight, "weight", (D, K), torch.float32, dev)
    _check(bias, "bias", (D,), torch.float32, dev)
    out_dt = x.dtype if out_dtype is None else out_dtype
    if y is None:
        y = torch.empty((B, D, L), dtype=out_dt, device=dev)
    _check(y, "y", (B, D, L), out_dt, dev)
    if return_final_state:
        if final_state is None:
            final_state = torch.empty((B, D, K), dtype=torch.float32, device=dev)
        _check(final_state, "final_state", (B, D, K), torch.float32, dev)
    st = lib().mamba_conv1d_fwd(_ptr(x), _ptr(weight), _ptr(bias), _ptr(y),
                                _ptr(final_state if return_final_state else None), B, D, L, K,
                                _dtype_code(x), _dtype_code(y), 1 if return_final_state else 0,
                                _stream(dev, stream))
    if st != 0:
        raise MambaError(st, "mamba_conv1d_fwd")
    return (y, final_state) if return_final_state else y


def conv1d_update(state, x, weight, bias=None, *, out_dtype=None, y=None, stream=None):
    """One decoding step of the convolution; `state` (B, D, K) fp32 (the K most
    recent inputs, oldest first) is updated in place.  x: (B, D).  Returns y (B, D)."""
    torch = _torch()
    if state.dim() != 3:
        raise ValueError("state must be (B, D, K)")
    B, D, K = state.shape
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    _dtype_code(x)
    _check(state, "state", (B, D, K), torch.float32, dev)
    _check(x, "x", (B, D), x.dtype, dev)
    _check(weight, "weight", (D, K), torch.float32, dev)
    _check(bias, "bias", (D,), torch.float32, dev)
    out_dt = x.dtype if out_dtype is None else out_dtype
    if y is None:
        y = torch.empty((B, D), dtype=out_dt, device=dev)
    _check(y, "y", (B, D), out_dt, dev)
    st = lib().mamba_conv1d_update(_ptr(state), _ptr(x), _ptr(weight), _ptr(bias), _ptr(y), B, D, K,
                                   _dtype_code(x), _dtype_code(y), _stream(dev, stream))
    if st != 0:
        raise MambaError(st, "mamba_conv1d_update")
    return y


def scan_bwd_workspace_size(B: int, D: int, N: int, L: int) -> int:
    n = lib().mamba_scan_bwd_workspace_size(B, D, N, L)
    if n == ctypes.c_size_t(-1).value:
        raise MambaError(-2, "mamba_scan_bwd_workspace_size")
    return n


def scan_bwd(u, delta, z, Bt, Ct, A, Dskip, delta_bias, dy, *, grad_dtype=None, delta_b=False,
             accurate_expm1=False, workspace=None, stream=None):
    """Gradients of scan_fwd (zero initial state) for output gradient dy (B, D, L).

    Returns a dict: du, ddelta, dz (B, D, L) in grad_dtype (dz None when z is
    None); dBt, dCt (B, N, L), dA (D, N), dDskip (D), ddelta_bias (D) fp32.
    """
    torch = _torch()
    if u.dim() != 3 or Bt.dim() != 3:
        raise ValueError("u must be (B, D, L) and Bt (B, N, L)")
    B, D, L = u.shape
    N = Bt.shape[1]
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    in_dt = u.dtype
    _dtype_code(u)
    for t, n, shp in ((u, "u", (B, D, L)), (delta, "delta", (B, D, L)), (z, "z", (B, D, L)),
                      (Bt, "Bt", (B, N, L)), (Ct, "Ct", (B, N, L))):
        _check(t, n, shp, in_dt, dev)
    _check(A, "A", (D, N), torch.float32, dev)
    _check(Dskip, "Dskip", (D,), torch.float32, dev)
    _check(delta_bias, "delta_bias", (D,), torch.float32, dev)
    gdt = dy.dtype if grad_dtype is None else grad_dtype
    _check(dy, "dy", (B, D, L), gdt, dev)
    out = {"du": torch.empty((B, D, L), dtype=gdt, device=dev), "ddelta": torch.empty((B, D, L), dtype=gdt, device=dev),
           "dz": torch.empty((B, D, L), dtype=gdt, device=dev) if z is not None else None,
           "dBt": torch.empty((B, N, L), dtype=torch.float32, device=dev),
           "dCt": torch.empty((B, N, L), dtype=torch.float32, device=dev),
           "dA": torch.empty((D, N), dtype=torch.float32, device=dev),
           "dDskip": torch.empty((D,), dtype=torch.float32, device=dev),
           "ddelta_bias": torch.empty((D,), dtype=torch.float32, device=dev)}
    wsb = scan_bwd_workspace_size(B, D, N, L)
    if workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    st = lib().mamba_scan_bwd(
        _ptr(u), _ptr(delta), _ptr(z), _ptr(Bt), _ptr(Ct), _ptr(A), _ptr(Dskip), _ptr(delta_bias), _ptr(dy),
        _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dz"]), _ptr(out["dBt"]), _ptr(out["dCt"]), _ptr(out["dA"]),
        _ptr(out["dDskip"]), _ptr(out["ddelta_bias"]), B, D, N, L, _dtype_code(u), _dtype_code(dy),
        (FLAG_DELTA_B if delta_b else 0) | (FLAG_ACCURATE_EXPM1 if accurate_expm1 else 0),
        _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(dev, stream))
    if st != 0:
        raise MambaError(st, "mamba_scan_bwd")
    return out
