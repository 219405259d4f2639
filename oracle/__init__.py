"""fp64 CPU oracle for the Mamba-1 selective scan and the single-token update.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``.  The GPU library never imports,
links or calls anything here, and this package imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, libm's exp/expm1/log1p,
no fast-math).  This module only marshals numpy arrays to it; every input is
first up-converted to float64, which is exact for the bf16 and fp32 values
the GPU sees.

Pages followed (titles and sections; each step is cited in ``oracle.c``):
  "Mamba 模型" (gaos6e.github.io) -- the full-step flowchart, nodes E, F and H to M;
  "Mamba 与状态空间模型" (world.lapla.si, plate F56) -- sections 03, 06, 07;
  "Mamba 状态空间模型架构深度解析" (pnsm.cn) -- ZOH, diagonal A;
  "Mamba模型：高效序列建模的新突破" (mhpn.cn) -- section 3.1, ZOH B-bar.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_LIB points the wrapper at another build of oracle.c (the sanitizer
# test's instrumented copy); it is then loaded as it is, never rebuilt.
_LIB = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

DISCRETIZATIONS = {"zoh": 0, "delta_b": 1}


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc -O2 (no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.environ.get("ORACLE_LIB") and (not os.path.exists(_LIB) or
                                                      os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            dp = ctypes.POINTER(ctypes.c_double)
            i64 = ctypes.c_int64
            lib.oracle_scan.argtypes = [i64, i64, i64, i64] + [dp] * 9 + [ctypes.c_int, dp, dp, ctypes.c_int]
            lib.oracle_scan.restype = ctypes.c_int
            lib.oracle_state_update.argtypes = [i64, i64, i64, dp] + [dp] * 8 + [ctypes.c_int, dp, ctypes.c_int]
            lib.oracle_state_update.restype = ctypes.c_int
            lib.oracle_scan_bwd.argtypes = [i64, i64, i64, i64] + [dp] * 8 + [ctypes.c_int] + [dp] * 9 + \
                [ctypes.c_int]
            lib.oracle_scan_bwd.restype = ctypes.c_int
            lib.oracle_conv1d.argtypes = [i64, i64, i64, i64, dp, dp, dp, dp, ctypes.c_int, dp, dp]
            lib.oracle_conv1d.restype = ctypes.c_int
            lib.oracle_conv1d_update.argtypes = [i64, i64, i64, dp, dp, dp, dp, ctypes.c_int, dp]
            lib.oracle_conv1d_update.restype = ctypes.c_int
            lib.oracle_softplus.argtypes = [ctypes.c_double]
            lib.oracle_softplus.restype = ctypes.c_double
            _lib = lib
    return _lib


def default_threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return max(1, min(16, os.cpu_count() or 1))


def _f64(a, shape=None):
    if a is None:
        return None
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError("expected shape %s, got %s" % (tuple(shape), a.shape))
    return a


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def softplus(x: float) -> float:
    return _load().oracle_softplus(float(x))


def scan(u, delta_raw, z, Bt, Ct, A, Dskip=None, delta_bias=None, h0=None,
         discretization: str = "zoh", nthreads: int | None = None):
    """Selective scan over (B, D, L).  Returns (y (B,D,L), final_state (B,D,N)), float64."""
    u = _f64(u)
    if u.ndim != 3:
        raise ValueError("u must be (B, D, L)")
    B, D, L = u.shape
    Bt = _f64(Bt)
    if Bt.ndim != 3 or Bt.shape[0] != B or Bt.shape[2] != L:
        raise ValueError("Bt must be (B, N, L)")
    N = Bt.shape[1]
    delta_raw = _f64(delta_raw, (B, D, L))
    z = _f64(z, (B, D, L))
    Ct = _f64(Ct, (B, N, L))
    A = _f64(A, (D, N))
    Dskip = _f64(Dskip, (D,))
    delta_bias = _f64(delta_bias, (D,))
    h0 = _f64(h0, (B, D, N))
    y = np.empty((B, D, L), dtype=np.float64)
    hN = np.empty((B, D, N), dtype=np.float64)
    rc = _load().oracle_scan(B, D, N, L, _ptr(u), _ptr(delta_raw), _ptr(z), _ptr(Bt), _ptr(Ct),
                             _ptr(A), _ptr(Dskip), _ptr(delta_bias), _ptr(h0),
                             DISCRETIZATIONS[discretization], _ptr(y), _ptr(hN),
                             nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_scan failed with %d" % rc)
    return y, hN


def state_update(state, u, delta_raw, z, Bt, Ct, A, Dskip=None, delta_bias=None,
                 discretization: str = "zoh", nthreads: int | None = None):
    """One decoding step.  state (B,D,N); u, delta_raw, z (B,D); Bt, Ct (B,N).

    Returns (y (B,D), new_state (B,D,N)) as float64; the input is not modified.
    """
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    if st.ndim != 3:
        raise ValueError("state must be (B, D, N)")
    B, D, N = st.shape
    u = _f64(u, (B, D))
    delta_raw = _f64(delta_raw, (B, D))
    z = _f64(z, (B, D))
    Bt = _f64(Bt, (B, N))
    Ct = _f64(Ct, (B, N))
    A = _f64(A, (D, N))
    Dskip = _f64(Dskip, (D,))
    delta_bias = _f64(delta_bias, (D,))
    y = np.empty((B, D), dtype=np.float64)
    rc = _load().oracle_state_update(B, D, N, _ptr(st), _ptr(u), _ptr(delta_raw), _ptr(z),
                                     _ptr(Bt), _ptr(Ct), _ptr(A), _ptr(Dskip), _ptr(delta_bias),
                                     DISCRETIZATIONS[discretization], _ptr(y),
                                     nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_state_update failed with %d" % rc)
    return y, st


def ssd_scan(x, delta_raw, z, Bt, Ct, A_head, Dskip=None, delta_bias=None, P: int = 64,
             discretization: str = "zoh", nthreads: int | None = None):
    """Mamba-2 layer (SSD) over x (B, H*P, L) with one scalar A per head.

    "Mamba 与状态空间模型" section 09 and "Mamba 状态空间模型架构深度解析"
    (Mamba-2): A is a scalar times the identity, so the layer is the same
    selective recurrence with A[d, n] = A_head[h] for every state n of every
    channel d of head h; the step size is shared by the head's P channels,
    which is what lets one lower-triangular matrix act on all of them.

    delta_raw (B, H, L), delta_bias (H) are per head; x, z (B, H*P, L);
    Bt, Ct (B, N, L); Dskip (H*P).  Returns (y (B, H*P, L), final_state
    (B, H*P, N)) as float64, by expanding the heads into the pinned scan.
    """
    x = _f64(x)
    if x.ndim != 3:
        raise ValueError("x must be (B, H*P, L)")
    B, D, L = x.shape
    if P < 1 or D % P:
        raise ValueError("H*P must be a multiple of P")
    H = D // P
    delta_raw = _f64(delta_raw, (B, H, L))
    A_head = _f64(A_head, (H,))
    N = _f64(Bt).shape[1]
    A = np.repeat(A_head, P)[:, None] * np.ones((1, N))
    dr = np.repeat(delta_raw, P, axis=1)
    bias = None if delta_bias is None else np.repeat(_f64(delta_bias, (H,)), P)
    return scan(x, dr, z, Bt, Ct, A, Dskip, bias, discretization=discretization, nthreads=nthreads)


def conv1d(x, w, bias=None, state0=None, activation: bool = True):
    """Causal depthwise convolution (+ SiLU) over (B, D, L); w is (D, K), tap i
    multiplies x[t - i].  Returns (y (B,D,L), final_state (B,D,K)), float64."""
    x = _f64(x)
    if x.ndim != 3:
        raise ValueError("x must be (B, D, L)")
    B, D, L = x.shape
    w = _f64(w)
    if w.ndim != 2 or w.shape[0] != D:
        raise ValueError("w must be (D, K)")
    K = w.shape[1]
    bias = _f64(bias, (D,))
    state0 = _f64(state0, (B, D, K))
    y = np.empty((B, D, L), dtype=np.float64)
    fs = np.empty((B, D, K), dtype=np.float64)
    rc = _load().oracle_conv1d(B, D, L, K, _ptr(x), _ptr(w), _ptr(bias), _ptr(state0), int(activation),
                               _ptr(y), _ptr(fs))
    if rc != 0:
        raise RuntimeError("oracle_conv1d failed with %d" % rc)
    return y, fs


def conv1d_update(state, x, w, bias=None, activation: bool = True):
    """One decoding step of the convolution.  state (B,D,K) (oldest first), x (B,D).
    Returns (y (B,D), new_state (B,D,K)) as float64; the input is not modified."""
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    if st.ndim != 3:
        raise ValueError("state must be (B, D, K)")
    B, D, K = st.shape
    x = _f64(x, (B, D))
    w = _f64(w, (D, K))
    bias = _f64(bias, (D,))
    y = np.empty((B, D), dtype=np.float64)
    rc = _load().oracle_conv1d_update(B, D, K, _ptr(st), _ptr(x), _ptr(w), _ptr(bias), int(activation), _ptr(y))
    if rc != 0:
        raise RuntimeError("oracle_conv1d_update failed with %d" % rc)
    return y, st


def scan_bwd(u, delta_raw, z, Bt, Ct, A, Dskip, delta_bias, dy, discretization: str = "zoh",
             nthreads: int | None = None):
    """Gradients of the scan for output gradient dy (B, D, L).

    Returns a dict of float64 arrays: du, ddelta_raw, dz (B, D, L; dz None when
    z is None), dBt, dCt (B, N, L), dA (D, N), dDskip (D), ddelta_bias (D).
    Dskip / delta_bias of None mean zeros (their gradients are still returned).
    """
    u = _f64(u)
    if u.ndim != 3:
        raise ValueError("u must be (B, D, L)")
    B, D, L = u.shape
    Bt = _f64(Bt)
    N = Bt.shape[1]
    delta_raw = _f64(delta_raw, (B, D, L))
    z = _f64(z, (B, D, L))
    Bt = _f64(Bt, (B, N, L))
    Ct = _f64(Ct, (B, N, L))
    A = _f64(A, (D, N))
    Dskip = _f64(Dskip, (D,))
    delta_bias = _f64(delta_bias, (D,))
    dy = _f64(dy, (B, D, L))
    out = {"du": np.empty((B, D, L)), "ddelta_raw": np.empty((B, D, L)),
           "dz": np.empty((B, D, L)) if z is not None else None,
           "dBt": np.empty((B, N, L)), "dCt": np.empty((B, N, L)), "dA": np.empty((D, N)),
           "dDskip": np.empty(D), "ddelta_bias": np.empty(D)}
    rc = _load().oracle_scan_bwd(B, D, N, L, _ptr(u), _ptr(delta_raw), _ptr(z), _ptr(Bt), _ptr(Ct), _ptr(A),
                                 _ptr(Dskip), _ptr(delta_bias), DISCRETIZATIONS[discretization], _ptr(dy),
                                 _ptr(out["du"]), _ptr(out["ddelta_raw"]), _ptr(out["dz"]), _ptr(out["dBt"]),
                                 _ptr(out["dCt"]), _ptr(out["dA"]), _ptr(out["dDskip"]), _ptr(out["ddelta_bias"]),
                                 nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_scan_bwd failed with %d" % rc)
    return out
