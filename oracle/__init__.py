"""fp64 CPU oracle for the KDA gated delta rule — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package.  The GPU library never loads it and shares no code with it.

What it computes (pages: "Kimi K3, explained", sections "How Kimi Delta Attention works,
step by step" and "The math"), per sequence and head, with the state S in R^{d_k x d_v}
(the page's d_v x d_k state, transposed):

    alpha_t = exp(g_t)                                    (per key channel)
    S_t     = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
    o_t     = S_t^T q_t                                   (read after the write)

``recurrence`` is the definition stepped token by token (the oracle proper); ``backward`` is
its reverse-mode derivative (the same token steps taken backwards); ``chunked``
is the chunked algebra in fp64 (used only to pin that the chunked form reaches the same
result); ``linear_attention`` is the page's contrast rule S <- S + k v^T.

Every pin that ties this oracle to the pages lives in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib_path() -> str:
    return os.path.join(_HERE, "_kda_oracle.so")


def build(verbose: bool = False) -> str:
    """Compile the C oracle with gcc (plain -O2, portable x86-64 code)."""
    import subprocess

    src = os.path.join(_HERE, "kda_oracle.c")
    out = lib_path()
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-o", tmp, src, "-lm", "-lpthread"]
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
            raise RuntimeError(f"oracle not built: {p} (run __graft_entry__.build())")
        L = ctypes.CDLL(p)
        dp, ip, i64 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64
        L.kda_oracle_recurrence.restype = ctypes.c_int
        L.kda_oracle_recurrence.argtypes = [dp, dp, dp, dp, dp, ip, i64, dp, dp, dp, i64, i64, i64, i64,
                                            ctypes.c_int]
        L.kda_oracle_recurrence_snap.restype = ctypes.c_int
        L.kda_oracle_recurrence_snap.argtypes = L.kda_oracle_recurrence.argtypes + [i64, ip, dp]
        L.kda_oracle_chunked.restype = ctypes.c_int
        L.kda_oracle_chunked.argtypes = [dp, dp, dp, dp, dp, ip, i64, dp, dp, dp, i64, i64, i64, i64,
                                         ctypes.c_int]
        L.kda_oracle_backward.restype = ctypes.c_int
        L.kda_oracle_backward.argtypes = [dp, dp, dp, dp, dp, ip, i64, dp, dp, dp, dp, dp, dp, dp, dp, dp, i64, i64,
                                          i64, ctypes.c_int]
        L.kda_oracle_linear_attention.restype = ctypes.c_int
        L.kda_oracle_linear_attention.argtypes = [dp, dp, dp, i64, i64, i64, dp, dp, dp]
        _LIB = L
    return _LIB


def default_threads() -> int:
    """Host threads the oracle uses: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data


def _prep(q, k, v, g, beta, cu, s0):
    q, k, v, g, beta, s0 = map(_f64, (q, k, v, g, beta, s0))
    T, H, dk = q.shape
    dv = v.shape[2]
    if g.shape == (T, H):
        # one log-decay per token and head (Gated DeltaNet): Diag(alpha_t) = alpha_t * I, the
        # same decay on every key channel
        g = np.ascontiguousarray(np.broadcast_to(g[:, :, None], (T, H, dk)))
    if k.shape != (T, H, dk) or g.shape != (T, H, dk) or v.shape[:2] != (T, H) or beta.shape != (T, H):
        raise ValueError("shape mismatch: q,k,g [T,H,dk], v [T,H,dv], beta [T,H]")
    cu = np.asarray([0, T] if cu is None else cu, dtype=np.int64)
    N = len(cu) - 1
    if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, end at T and be non-decreasing")
    if s0 is not None and s0.shape != (N, H, dk, dv):
        raise ValueError(f"s0 must be [N,H,dk,dv]={(N, H, dk, dv)}, got {s0.shape}")
    return q, k, v, g, beta, np.ascontiguousarray(cu), s0, T, H, dk, dv, N


def recurrence(q, k, v, g, beta, cu=None, s0=None, *, threads=None, vcols=0, snapshot_every=0):
    """Token-by-token fp64 recurrence.  Inputs [T,H,d] (packed sequences per ``cu``),
    g = log(alpha) [T,H,dk] (one decay per key channel) or [T,H] (one per head), beta [T,H],
    s0 [N,H,dk,dv] or None.  Returns (o, sT), plus the state snapshots [S,H,dk,dv] when
    snapshot_every > 0: the state after every snapshot_every tokens of each sequence, in
    sequence order."""
    q, k, v, g, beta, cu, s0, T, H, dk, dv, N = _prep(q, k, v, g, beta, cu, s0)
    o = np.zeros((T, H, dv), np.float64)
    sT = np.zeros((N, H, dk, dv), np.float64)
    snap_cu = np.zeros(N + 1, np.int64)
    if snapshot_every > 0:
        snap_cu[1:] = np.cumsum(np.diff(cu) // snapshot_every)
    snaps = np.zeros((int(snap_cu[-1]), H, dk, dv), np.float64)
    rc = _lib().kda_oracle_recurrence_snap(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), cu.ctypes.data, N,
                                           _ptr(s0), o.ctypes.data, sT.ctypes.data, H, dk, dv, int(vcols),
                                           threads or default_threads(), int(snapshot_every), snap_cu.ctypes.data,
                                           snaps.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"kda_oracle_recurrence failed ({rc})")
    return (o, sT, snaps) if snapshot_every > 0 else (o, sT)


def backward(q, k, v, g, beta, cu=None, s0=None, *, d_o, d_sT=None, threads=None):
    """Reverse-mode derivative of ``recurrence`` in fp64.  ``d_o`` [T,H,dv] is dL/do and ``d_sT``
    [N,H,dk,dv] (or None: zero) is dL/dS_T.  Returns (dq, dk, dv, dg, dbeta, ds0): dL/d of each
    input, with dg = dL/d(log alpha) in g's own shape ([T,H,dk], or [T,H] for one decay per head,
    the sum over key channels) and ds0 = dL/dS_0 [N,H,dk,dv] (returned also when s0 is None)."""
    head_gate = np.ndim(g) == 2
    q, k, v, g, beta, cu, s0, T, H, dk, dv, N = _prep(q, k, v, g, beta, cu, s0)
    d_o, d_sT = _f64(d_o), _f64(d_sT)
    if d_o.shape != (T, H, dv) or (d_sT is not None and d_sT.shape != (N, H, dk, dv)):
        raise ValueError("d_o must be [T,H,dv] and d_sT [N,H,dk,dv]")
    dq, dk_, dg = (np.zeros((T, H, dk), np.float64) for _ in range(3))
    dv_ = np.zeros((T, H, dv), np.float64)
    db = np.zeros((T, H), np.float64)
    ds0 = np.zeros((N, H, dk, dv), np.float64)
    rc = _lib().kda_oracle_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), cu.ctypes.data, N, _ptr(s0),
                                    _ptr(d_o), _ptr(d_sT), dq.ctypes.data, dk_.ctypes.data, dv_.ctypes.data,
                                    dg.ctypes.data, db.ctypes.data, ds0.ctypes.data, H, dk, dv,
                                    threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"kda_oracle_backward failed ({rc})")
    return dq, dk_, dv_, (dg.sum(-1) if head_gate else dg), db, ds0


def prologue(q, k, beta_logits, gate_in, gate_scale):
    """The input prologue of the DeltaNet family ("Kimi K3, explained", "How Kimi Delta Attention
    works, step by step"), in fp64: queries and keys L2-normalised per token and head (a zero
    vector stays zero), beta = sigmoid(logit), g = log(alpha) = -gate_scale * softplus(a).
    Returns (q, k, beta, g)."""
    q, k, b, a = (np.asarray(x, np.float64) for x in (q, k, beta_logits, gate_in))

    def unit(x):
        n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        return np.divide(x, n, out=np.zeros_like(x), where=n > 0)

    beta = 1.0 / (1.0 + np.exp(-b))
    g = -gate_scale * (np.maximum(a, 0.0) + np.log1p(np.exp(-np.abs(a))))
    return unit(q), unit(k), beta, g


def chunked(q, k, v, g, beta, cu=None, s0=None, *, chunk=16, threads=None):
    """fp64 chunked algebra (the form the GPU path organises its work in)."""
    q, k, v, g, beta, cu, s0, T, H, dk, dv, N = _prep(q, k, v, g, beta, cu, s0)
    o = np.zeros((T, H, dv), np.float64)
    sT = np.zeros((N, H, dk, dv), np.float64)
    rc = _lib().kda_oracle_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), cu.ctypes.data, N,
                                   _ptr(s0), o.ctypes.data, sT.ctypes.data, H, dk, dv, int(chunk),
                                   threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"kda_oracle_chunked failed ({rc})")
    return o, sT


def decode_step(q, k, v, g, beta, s0, *, threads=None):
    """One token for each of N sequences: q,k,g [N,H,dk], v [N,H,dv], beta [N,H], s0 [N,H,dk,dv]."""
    N = q.shape[0]
    return recurrence(q, k, v, g, beta, np.arange(N + 1), s0, threads=threads)


def linear_attention(q, k, v, s0=None):
    """Contrast rule (no erase, no decay) for one head: q,k [T,dk], v [T,dv]."""
    q, k, v, s0 = map(_f64, (q, k, v, s0))
    T, dk = q.shape
    dv = v.shape[1]
    o = np.zeros((T, dv), np.float64)
    sT = np.zeros((dk, dv), np.float64)
    rc = _lib().kda_oracle_linear_attention(_ptr(q), _ptr(k), _ptr(v), T, dk, dv, _ptr(s0), o.ctypes.data,
                                            sT.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"kda_oracle_linear_attention failed ({rc})")
    return o, sT
