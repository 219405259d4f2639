"""Seeded synthetic workloads for the selective scan and the decode step.

This module holds random draws, shapes and dtype plumbing only -- none of the
scan's arithmetic.  It serves both the GPU path (tests, benchmark, smoke
check) and the fp64 oracle, so both see bit-identical inputs.

Shapes and distributions follow the workloads the pages describe: a state of
N = 16 numbers per channel and A initialised to -1 ... -16 ("Mamba 与状态空间
模型", sections 03 and 04); a 2.8B-model layer of 5,120 channels (section 03);
prompt 2,048 + 128 generated tokens at batch 128 for decoding (section 08);
sequences up to 2^19 at batch 1 for the scan ("Mamba论文研读笔记", 4.5 table,
efficiency row).

Draw recipe (identical for every workload, all Generators are numpy PCG64):
  * dt_d ~ log-uniform[1e-3, 1e-1] (fp64), delta_bias_d = log(expm1(dt_d)) rounded to
    fp32, so that softplus(delta_bias_d) = dt_d;
  * Dskip_d = 1 (tiny fp32 workload) or ~ N(0, 1) rounded to fp32;
  * A[d, n] = -(n + 1);
  * delta_raw, u, z (B, D, L) and B_t, C_t (B, N, L) ~ N(0, 1): fp32 draws, rounded
    to nearest-even bf16 for the bf16 workloads;
  * big arrays are drawn in fixed blocks of 2^22 elements, block k of array a
    from SeedSequence([seed, a, k]), so the values do not depend on the number
    of threads used to draw them.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import hashlib
import os

import numpy as np

BLOCK = 1 << 22

# Array ids used in the seed tree (kept fixed: changing them changes every input).
_ID_PARAMS, _ID_DELTA, _ID_U, _ID_Z, _ID_B, _ID_C, _ID_STATE = range(7)
_ID_CONV_X, _ID_CONV_PARAMS, _ID_CONV_STATE = range(7, 10)
_ID_SSD_PARAMS, _ID_SSD_X, _ID_SSD_DT, _ID_SSD_Z, _ID_SSD_B, _ID_SSD_C = range(10, 16)


@dataclasses.dataclass(frozen=True)
class ScanConfig:
    name: str
    B: int
    D: int
    N: int
    L: int
    dtype: str          # "f32" or "bf16": dtype of u, delta_raw, z, B_t, C_t and y
    seed: int
    dskip: str          # "ones" or "normal"
    final_state: bool

    @property
    def elements(self) -> int:
        return self.B * self.D * self.L

    @property
    def updates(self) -> int:
        return self.B * self.D * self.L * self.N

    def algorithmic_bytes(self) -> int:
        """Bytes the method must move: every input once, y once, final state once."""
        e = 4 if self.dtype == "f32" else 2
        b = 3 * self.B * self.D * self.L * e          # u, delta_raw, z
        b += 2 * self.B * self.N * self.L * e         # B_t, C_t
        b += self.D * self.N * 4 + 2 * self.D * 4     # A, Dskip, delta_bias
        b += self.B * self.D * self.L * e             # y
        if self.final_state:
            b += self.B * self.D * self.N * 4
        return b


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    layers: int
    steps: int
    B: int
    D: int
    N: int
    seed: int
    state_sigma: float = 0.1

    def bytes_per_layer_step(self) -> int:
        """State read + written in place, u/delta/z/y (bf16), B_t/C_t (bf16), A/Dskip/bias (fp32)."""
        st = self.B * self.D * self.N * 4
        return 2 * st + 4 * self.B * self.D * 2 + 2 * self.B * self.N * 2 + self.D * self.N * 4 + 2 * self.D * 4


SCAN_CONFIGS = {
    "tiny_fp32": ScanConfig("tiny_fp32", 1, 16, 16, 256, "f32", 1000, "ones", False),
    "mamba130m_layer": ScanConfig("mamba130m_layer", 8, 1536, 16, 2048, "bf16", 1001, "normal", False),
    "mamba2.8b_layer": ScanConfig("mamba2.8b_layer", 4, 5120, 16, 2048, "bf16", 1002, "normal", True),
    "long_b1": ScanConfig("long_b1", 1, 4096, 16, 131072, "bf16", 1003, "normal", False),
}
DECODE_CONFIGS = {
    "decode48": DecodeConfig("decode48", 48, 128, 128, 4096, 16, 1004),
}


# ----------------------------------------------------------------------------- dtype plumbing
def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f32(a) -> np.ndarray:
    """float32 view of an input array, whether it is stored as float32 or as bf16 bits."""
    a = np.asarray(a)
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a.astype(np.float32, copy=False)


def sha256(a) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()


# ----------------------------------------------------------------------------- drawing
def _threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    n = int(env) if env and env.isdigit() and int(env) > 0 else (os.cpu_count() or 1)
    return max(1, min(16, n))


def _normal_f32(seed_path, count: int) -> np.ndarray:
    """`count` standard-normal float32 draws, block k drawn from SeedSequence(seed_path + [k])."""
    out = np.empty(count, dtype=np.float32)
    nblk = (count + BLOCK - 1) // BLOCK

    def fill(k):
        lo, hi = k * BLOCK, min(count, (k + 1) * BLOCK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed_path) + [k])))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    if nblk <= 1:
        if count:
            fill(0)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def _params(seed_path, D: int, N: int, dskip: str):
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed_path) + [_ID_PARAMS])))
    dt = np.exp(g.uniform(np.log(1e-3), np.log(1e-1), size=D))          # fp64
    delta_bias = np.log(np.expm1(dt)).astype(np.float32)
    if dskip == "ones":
        Dskip = np.ones(D, dtype=np.float32)
    else:
        Dskip = g.standard_normal(D).astype(np.float32)
    A = np.broadcast_to(-(np.arange(N, dtype=np.float32) + 1.0), (D, N)).copy()
    return A, Dskip, delta_bias, dt


def scan_inputs(cfg: ScanConfig) -> dict:
    """All inputs of one scan workload.  bf16 arrays are uint16 bit patterns."""
    s = [cfg.seed]
    A, Dskip, delta_bias, dt = _params(s, cfg.D, cfg.N, cfg.dskip)
    big = (cfg.B, cfg.D, cfg.L)
    bc = (cfg.B, cfg.N, cfg.L)
    out = {
        "A": A, "Dskip": Dskip, "delta_bias": delta_bias, "dt": dt,
        "delta_raw": _store(_normal_f32(s + [_ID_DELTA], int(np.prod(big))), cfg.dtype).reshape(big),
        "u": _store(_normal_f32(s + [_ID_U], int(np.prod(big))), cfg.dtype).reshape(big),
        "z": _store(_normal_f32(s + [_ID_Z], int(np.prod(big))), cfg.dtype).reshape(big),
        "Bt": _store(_normal_f32(s + [_ID_B], int(np.prod(bc))), cfg.dtype).reshape(bc),
        "Ct": _store(_normal_f32(s + [_ID_C], int(np.prod(bc))), cfg.dtype).reshape(bc),
    }
    return out


def custom_scan_inputs(B: int, D: int, N: int, L: int, dtype: str, seed: int, dskip: str = "normal") -> dict:
    """Same recipe at an arbitrary shape (ragged and edge-case parity tests)."""
    return scan_inputs(ScanConfig("custom", B, D, N, L, dtype, seed, dskip, True))


def decode_layer_params(cfg: DecodeConfig, layer: int):
    """(A, Dskip, delta_bias, state0) of one layer; state0 ~ N(0, sigma) fp32."""
    s = [cfg.seed, layer]
    A, Dskip, delta_bias, _ = _params(s, cfg.D, cfg.N, "normal")
    st = _normal_f32(s + [_ID_STATE], cfg.B * cfg.D * cfg.N) * np.float32(cfg.state_sigma)
    return A, Dskip, delta_bias, st.reshape(cfg.B, cfg.D, cfg.N)


def decode_step_inputs(cfg: DecodeConfig, layer: int, step: int) -> dict:
    """bf16 u, delta_raw, z (B, D) and B_t, C_t (B, N) of one token at one layer."""
    s = [cfg.seed, layer, 1000 + step]
    bd, bn = (cfg.B, cfg.D), (cfg.B, cfg.N)
    return {
        "delta_raw": f32_to_bf16_bits(_normal_f32(s + [_ID_DELTA], cfg.B * cfg.D)).reshape(bd),
        "u": f32_to_bf16_bits(_normal_f32(s + [_ID_U], cfg.B * cfg.D)).reshape(bd),
        "z": f32_to_bf16_bits(_normal_f32(s + [_ID_Z], cfg.B * cfg.D)).reshape(bd),
        "Bt": f32_to_bf16_bits(_normal_f32(s + [_ID_B], cfg.B * cfg.N)).reshape(bn),
        "Ct": f32_to_bf16_bits(_normal_f32(s + [_ID_C], cfg.B * cfg.N)).reshape(bn),
    }


# ----------------------------------------------------------------------------- causal conv1d + SiLU
@dataclasses.dataclass(frozen=True)
class ConvConfig:
    """Causal depthwise conv1d + SiLU over x (B, D, L) with K taps per channel."""
    name: str
    B: int
    D: int
    L: int
    K: int
    dtype: str          # dtype of x and y
    seed: int

    @property
    def elements(self) -> int:
        return self.B * self.D * self.L

    def algorithmic_bytes(self) -> int:
        """x read once, y written once, taps and bias read once, final state written."""
        e = 2 if self.dtype == "bf16" else 4
        return self.elements * 2 * e + self.D * (self.K + 1) * 4 + self.B * self.D * self.K * 4


@dataclasses.dataclass(frozen=True)
class ConvUpdateConfig:
    """One-token conv updates: `layers` layers x `steps` steps at (B, D, K)."""
    name: str
    B: int
    D: int
    K: int
    layers: int
    steps: int
    seed: int

    def bytes_per_layer_step(self) -> int:
        """state read + written (fp32), x read and y written (bf16), taps and bias."""
        rows = self.B * self.D
        return rows * self.K * 4 * 2 + rows * 2 * 2 + self.D * (self.K + 1) * 4


# The scan's 2.8B layer shape (the conv feeds u to it); the decode shape of the
# 48-layer state update.  Taps and bias ~ U(-1/2, 1/2) (the usual uniform
# initialisation bound 1/sqrt(fan-in) for K = 4 taps), x ~ N(0, 1).
CONV_CONFIGS = {
    "conv_2.8b_layer": ConvConfig("conv_2.8b_layer", 4, 5120, 2048, 4, "bf16", 1005),
}
CONV_UPDATE_CONFIGS = {
    "conv_decode48": ConvUpdateConfig("conv_decode48", 128, 4096, 4, 48, 128, 1006),
}


def _conv_params(seed_path, D: int, K: int):
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed_path) + [_ID_CONV_PARAMS])))
    w = g.uniform(-0.5, 0.5, size=(D, K)).astype(np.float32)
    bias = g.uniform(-0.5, 0.5, size=D).astype(np.float32)
    return w, bias


def conv_inputs(B: int, D: int, L: int, K: int, dtype: str, seed: int) -> dict:
    """x (B, D, L) in `dtype` (bf16 as uint16 bit patterns), w (D, K) and bias (D) fp32."""
    x = _normal_f32([seed, _ID_CONV_X], B * D * L).reshape(B, D, L)
    w, bias = _conv_params([seed], D, K)
    return {"x": _store(x, dtype), "w": w, "bias": bias}


def conv_update_layer(cfg: ConvUpdateConfig, layer: int):
    """(w, bias, state0) of one layer; state0 ~ N(0, 1) fp32 rounded through bf16
    (the state holds past inputs, which are bf16 values)."""
    w, bias = _conv_params([cfg.seed, layer], cfg.D, cfg.K)
    st = _normal_f32([cfg.seed, layer, _ID_CONV_STATE], cfg.B * cfg.D * cfg.K).reshape(cfg.B, cfg.D, cfg.K)
    return w, bias, as_f32(f32_to_bf16_bits(st))


def conv_update_step(cfg: ConvUpdateConfig, layer: int, step: int) -> np.ndarray:
    """x (B, D) bf16 bit patterns of one layer at one step."""
    x = _normal_f32([cfg.seed, layer, step, _ID_CONV_X], cfg.B * cfg.D).reshape(cfg.B, cfg.D)
    return f32_to_bf16_bits(x)


# ----------------------------------------------------------------------------- Mamba-2 (SSD)
@dataclasses.dataclass(frozen=True)
class SsdConfig:
    """Mamba-2 layer: H heads of P channels (D = H P), one scalar A and one step
    size per head, N states per channel shared B_t / C_t ("Mamba 与状态空间模型"
    section 09: N = 128 in the released models)."""
    name: str
    B: int
    H: int
    P: int
    N: int
    L: int
    seed: int
    gate: bool

    @property
    def D(self) -> int:
        return self.H * self.P

    @property
    def elements(self) -> int:
        return self.B * self.D * self.L

    def algorithmic_bytes(self, out_bytes: int = 2) -> int:
        """x (and z) read, y written, delta (B, H, L) and B_t / C_t read, all bf16;
        A, delta bias per head and D per channel read."""
        per = 2 * (2 if self.gate else 1) + out_bytes
        return (self.elements * per + self.B * self.H * self.L * 2 + 2 * self.B * self.N * self.L * 2
                + self.H * 2 * 4 + self.D * 4)


# The 2.8B-layer channel count (D = 5,120) cut into 80 heads of 64 channels,
# N = 128, batch 4, 2,048 tokens, gated.
SSD_CONFIGS = {
    "ssd_2.7b_layer": SsdConfig("ssd_2.7b_layer", 4, 80, 64, 128, 2048, 1007, True),
}


def ssd_inputs(B: int, H: int, P: int, N: int, L: int, seed: int, gate: bool = True) -> dict:
    """x, z (B, H P, L), delta_raw (B, H, L), B_t, C_t (B, N, L) ~ N(0, 1) as bf16 bit
    patterns; per head dt ~ log-uniform[1e-3, 1e-1] with delta_bias = log(expm1(dt))
    and A = -U[1, 16]; Dskip (H P) ~ N(0, 1); all fp32."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _ID_SSD_PARAMS])))
    dt = np.exp(g.uniform(np.log(1e-3), np.log(1e-1), size=H))
    delta_bias = np.log(np.expm1(dt)).astype(np.float32)
    A = (-g.uniform(1.0, 16.0, size=H)).astype(np.float32)
    Dskip = g.standard_normal(H * P).astype(np.float32)
    D = H * P
    big, bc = (B, D, L), (B, N, L)
    out = {
        "A": A, "Dskip": Dskip, "delta_bias": delta_bias, "dt": dt,
        "x": f32_to_bf16_bits(_normal_f32([seed, _ID_SSD_X], B * D * L)).reshape(big),
        "delta_raw": f32_to_bf16_bits(_normal_f32([seed, _ID_SSD_DT], B * H * L)).reshape(B, H, L),
        "Bt": f32_to_bf16_bits(_normal_f32([seed, _ID_SSD_B], B * N * L)).reshape(bc),
        "Ct": f32_to_bf16_bits(_normal_f32([seed, _ID_SSD_C], B * N * L)).reshape(bc),
        "z": f32_to_bf16_bits(_normal_f32([seed, _ID_SSD_Z], B * D * L)).reshape(big) if gate else None,
    }
    return out
