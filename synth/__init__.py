"""Seeded synthetic inputs for the KDA workloads (shared by the GPU path and the oracle).

Holds no arithmetic of the method: it draws queries, keys, values, write strengths
beta, per-channel log-decays g = log(alpha), carried states and segment lengths, with
the shapes and value distributions of the workloads the pages describe (head size
d_k = d_v = 128 as in Kimi K3's published configuration, contexts up to 2^20 tokens,
append-prefill segments).  The generator is a counter-based SplitMix64 stream in
``synth.c`` (built to ``_synth.so``); element i of a tensor depends only on
(seed, tensor id, i), so slices regenerate exactly.

Storage dtypes: ``"f32"`` -> numpy float32, ``"bf16"`` -> numpy uint16 holding bfloat16
bits (round-to-nearest-even from the fp32 value), ``"f64"`` -> float64.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

K_NORMAL, K_UNIT_ROWS, K_SIGMOID_NORMAL, K_LOGDECAY_SOFTPLUS, K_LOGDECAY_RATE, K_UNIFORM, K_UNIFORM_INT = range(7)
_OUT = {"f64": (0, np.float64), "f32": (1, np.float32), "bf16": (2, np.uint16), "i32": (3, np.int32)}

# tensor ids inside one workload's stream
TID_Q, TID_K, TID_V, TID_BETA, TID_G, TID_S0, TID_RATE, TID_LENS = 1, 2, 3, 4, 5, 6, 7, 8
TID_DO, TID_DST = 9, 10


def lib_path() -> str:
    return os.path.join(_HERE, "_synth.so")


def build(verbose: bool = False) -> str:
    """Compile ``synth.c`` with gcc (plain -O2, portable x86-64 code)."""
    import subprocess

    out = lib_path()
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-D_DEFAULT_SOURCE", "-o", tmp,
           os.path.join(_HERE, "synth.c"), "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _lib():
    global _LIB
    if _LIB is None:
        p = lib_path()
        if not os.path.exists(p):
            raise RuntimeError(f"synthetic-input generator not built: {p} (run __graft_entry__.build())")
        L = ctypes.CDLL(p)
        L.synth_fill.restype = ctypes.c_int
        L.synth_fill.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                 ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_double,
                                 ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
        L.synth_uniform_raw.restype = None
        L.synth_uniform_raw.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                        ctypes.c_void_p]
        L.synth_mix64.restype = ctypes.c_uint64
        L.synth_mix64.argtypes = [ctypes.c_uint64]
        _LIB = L
    return _LIB


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def fill(kind: int, seed: int, tid: int, shape, dtype: str = "f64", *, offset: int = 0, row_len: int = 0,
         heads: int = 0, p0: float = 0.0, p1: float = 0.0, tid2: int = 0, threads: int | None = None) -> np.ndarray:
    code, npdt = _OUT[dtype]
    out = np.empty(shape, dtype=npdt)
    rc = _lib().synth_fill(kind, seed, tid, tid2, offset, out.size, row_len, heads, p0, p1, code,
                           out.ctypes.data, threads or default_threads())
    if rc != 0:
        raise ValueError(f"synth_fill rejected kind={kind} shape={shape} offset={offset} row_len={row_len}")
    return out


def uniform_raw(seed: int, tid: int, start: int, count: int) -> np.ndarray:
    out = np.empty(count, np.float64)
    _lib().synth_uniform_raw(seed, tid, start, count, out.ctypes.data)
    return out


def mix64(z: int) -> int:
    return int(_lib().synth_mix64(z))


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of a stored tensor to float64 (what the oracle consumes)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


# ----------------------------------------------------------------------------------------------
# Workload recipes
# ----------------------------------------------------------------------------------------------
@dataclass
class Gate:
    """Per-channel log-decay recipe: g = -scale*softplus(N(0,1)) ("softplus"), or
    g = -softplus(N(0,1)) * r[h,c] with r ~ U(lo, hi) drawn once per (head, channel) ("rate")."""
    kind: str = "softplus"
    scale: float = 0.1
    lo: float = 0.001
    hi: float = 0.1


@dataclass
class Workload:
    name: str
    seed: int
    H: int
    dk: int
    dv: int
    dtype: str  # storage dtype of q, k, v, beta
    chunk: int = 64
    B: int = 1
    T: int = 0
    lengths: list = field(default_factory=list)  # varlen segment lengths (append-prefill)
    s0_std: float = 0.0  # 0 -> no initial state (zeros)
    gate: Gate = field(default_factory=Gate)
    q_unit: bool = True
    v_std: float = 1.0  # v ~ N(0, v_std^2)
    decode_steps: int = 0
    decode_N: int = 0


def gen_tokens(w: Workload, T: int, *, offset_tokens: int = 0, q_unit: bool | None = None, threads=None):
    """q, k, v, g, beta for T packed tokens x H heads (token-major [T, H, d])."""
    H, dk, dv, dt = w.H, w.dk, w.dv, w.dtype
    qu = w.q_unit if q_unit is None else q_unit
    off_k, off_v, off_h = offset_tokens * H * dk, offset_tokens * H * dv, offset_tokens * H
    if qu:
        q = fill(K_UNIT_ROWS, w.seed, TID_Q, (T, H, dk), dt, offset=off_k, row_len=dk, threads=threads)
    else:
        q = fill(K_NORMAL, w.seed, TID_Q, (T, H, dk), dt, offset=off_k, p0=1.0, threads=threads)
    k = fill(K_UNIT_ROWS, w.seed, TID_K, (T, H, dk), dt, offset=off_k, row_len=dk, threads=threads)
    v = fill(K_NORMAL, w.seed, TID_V, (T, H, dv), dt, offset=off_v, p0=w.v_std, threads=threads)
    beta = fill(K_SIGMOID_NORMAL, w.seed, TID_BETA, (T, H), dt, offset=off_h, threads=threads)
    if w.gate.kind == "softplus":
        g = fill(K_LOGDECAY_SOFTPLUS, w.seed, TID_G, (T, H, dk), "f32", offset=off_k, p0=w.gate.scale,
                 threads=threads)
    else:
        g = fill(K_LOGDECAY_RATE, w.seed, TID_G, (T, H, dk), "f32", offset=off_k, row_len=dk, heads=H,
                 p0=w.gate.lo, p1=w.gate.hi, tid2=TID_RATE, threads=threads)
    return q, k, v, g, beta


def gen_raw_tokens(w: Workload, T: int, *, offset_tokens: int = 0, gate_head: bool = False, threads=None):
    """Raw projections for the fused input prologue: q, k ~ N(0, 2^2) (not normalised),
    v ~ N(0, 1), beta logits ~ N(0, 1) (all stored in w.dtype), gate inputs a ~ N(0, 1) fp32,
    [T, H, dk] or [T, H] with one per head.  Returns (q, k, v, a, beta_logits)."""
    H, dk, dv, dt = w.H, w.dk, w.dv, w.dtype
    off_k, off_v, off_h = offset_tokens * H * dk, offset_tokens * H * dv, offset_tokens * H
    q = fill(K_NORMAL, w.seed, TID_Q, (T, H, dk), dt, offset=off_k, p0=2.0, threads=threads)
    k = fill(K_NORMAL, w.seed, TID_K, (T, H, dk), dt, offset=off_k, p0=2.0, threads=threads)
    v = fill(K_NORMAL, w.seed, TID_V, (T, H, dv), dt, offset=off_v, p0=1.0, threads=threads)
    beta = fill(K_NORMAL, w.seed, TID_BETA, (T, H), dt, offset=off_h, p0=1.0, threads=threads)
    if gate_head:
        a = fill(K_NORMAL, w.seed, TID_G, (T, H), "f32", offset=off_h, p0=1.0, threads=threads)
    else:
        a = fill(K_NORMAL, w.seed, TID_G, (T, H, dk), "f32", offset=off_k, p0=1.0, threads=threads)
    return q, k, v, a, beta


def gen_state(w: Workload, N: int, threads=None):
    """Carried fp32 state [N, H, dk, dv] ~ N(0, s0_std^2), or None for a zero state."""
    if w.s0_std <= 0:
        return None
    return fill(K_NORMAL, w.seed, TID_S0, (N, w.H, w.dk, w.dv), "f32", p0=w.s0_std, threads=threads)


def gen_cotangents(w: Workload, T: int, N: int, threads=None):
    """Upstream gradients of a loss for the backward pass: dL/do [T, H, dv] and dL/dS_T
    [N, H, dk, dv], both fp32 ~ N(0, 1)."""
    d_out = fill(K_NORMAL, w.seed, TID_DO, (T, w.H, w.dv), "f32", p0=1.0, threads=threads)
    d_sT = fill(K_NORMAL, w.seed, TID_DST, (N, w.H, w.dk, w.dv), "f32", p0=1.0, threads=threads)
    return d_out, d_sT


def gen_lengths(w: Workload, N: int, lo: int, hi: int) -> list:
    return [int(x) for x in fill(K_UNIFORM_INT, w.seed, TID_LENS, (N,), "f64", p0=lo, p1=hi)]


def cu_seqlens(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, np.int64))]).astype(np.int32)


# The five workloads (seed 75000 + index) plus the 64K-token prefill the headline metric is quoted on.
def workload(name: str) -> Workload:
    if name == "tiny":
        return Workload("tiny", 75000, H=2, dk=16, dv=16, dtype="f32", chunk=16, B=1, T=64)
    if name == "prefill":
        return Workload("prefill", 75001, H=32, dk=128, dv=128, dtype="bf16", chunk=64, B=1, T=8192)
    if name == "decode":
        return Workload("decode", 75002, H=32, dk=128, dv=128, dtype="bf16", s0_std=0.02, q_unit=False,
                        decode_steps=1000, decode_N=256)
    if name == "varlen":
        w = Workload("varlen", 75003, H=32, dk=128, dv=128, dtype="bf16", chunk=64, s0_std=0.02)
        w.lengths = gen_lengths(w, 8, 1024, 32768)
        w.T = sum(w.lengths)
        return w
    if name == "long":
        return Workload("long", 75004, H=32, dk=128, dv=128, dtype="bf16", chunk=64, B=1, T=1 << 20,
                        gate=Gate("rate", lo=0.001, hi=0.1), decode_steps=4096, decode_N=1)
    if name == "metric":
        return Workload("metric", 75005, H=32, dk=128, dv=128, dtype="bf16", chunk=64, B=1, T=65536)
    raise KeyError(name)


WORKLOADS = ("tiny", "prefill", "decode", "varlen", "long", "metric")
