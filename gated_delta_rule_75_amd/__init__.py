"""MI355X (gfx950) Kimi Delta Attention: chunked prefill, append-prefill and decode.

Thin Python binding over the C ABI in ``include/kda.h`` (library ``_kda.so``).  This
module only checks and marshals torch tensors (device memory) and the current HIP stream;
every step of the computation runs in the library's HIP kernels.

Per sequence and head, with state S in R^{d_k x d_v} and alpha = exp(g) per key channel
("Kimi K3, explained", "The math", gated delta rule equation, transposed):
    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import KdaError  # noqa: F401

__all__ = ["prefill_chunked", "append_prefill", "decode_step", "chunked_backward", "workspace_size", "is_supported",
           "version", "KdaError", "kernel_timing"]

_DT = {torch.float32: _lib.KDA_F32, torch.bfloat16: _lib.KDA_BF16}


def version() -> str:
    return _lib.load().kda_version().decode()


def is_supported(op: int, dtype: torch.dtype, dk: int, dv: int, chunk: int = 64) -> bool:
    return bool(_lib.load().kda_is_supported(op, _DT[dtype], dk, dv, chunk))


def workspace_size(op: int, n: int, t: int, h: int, dk: int, dv: int, dtype: torch.dtype, chunk: int) -> int:
    ws = _lib.load().kda_workspace_size(op, n, t, h, dk, dv, _DT[dtype], chunk)
    if ws == 2 ** 64 - 1:
        raise KdaError(_lib.KDA_ERR_UNSUPPORTED, f"unsupported op={op} dtype={dtype} dk={dk} dv={dv} chunk={chunk}")
    return int(ws)


class kernel_timing:
    """Context manager: per-kernel HIP-event timings of every library kernel launched inside it
    (on the calling thread).  After exit, ``records`` is a list of (kernel name, ms) in launch
    order; exiting waits for the recorded events."""

    MAX_RECORDS = 1 << 16

    def __init__(self):
        self.records = []

    def __enter__(self):
        _lib.check(_lib.load().kda_timing_begin())
        return self

    def __exit__(self, *exc):
        import ctypes

        ids = (ctypes.c_int32 * self.MAX_RECORDS)()
        ms = (ctypes.c_float * self.MAX_RECORDS)()
        n = _lib.load().kda_timing_end(ids, ms, self.MAX_RECORDS)
        if n < 0:
            _lib.check(n)
        self.records = [(_lib.KERNEL_NAMES.get(ids[i], str(ids[i])), float(ms[i]))
                        for i in range(min(n, self.MAX_RECORDS))]
        return False


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(t, name, dtype=None, shape=None, device=None):
    # fast path: a plain tensor that passes every test (the checks below raise with a message);
    # get_device() is an int (-1 on the CPU), cheaper than building the tensor's device object
    if type(t) is torch.Tensor:
        di = t.get_device()
        if (di >= 0 and (device is None or di == device.index) and (dtype is None or t.dtype == dtype)
                and (shape is None or t.shape == shape) and t.is_contiguous()):
            return
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


# torch's raw accessor of the current stream handle (no Stream object per call: about 0.1 us
# against 1.9 us for torch.cuda.current_stream(device).cuda_stream); the public call otherwise
_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device):
    if _RAW_STREAM is not None:
        return _RAW_STREAM(device.index if device.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


def _gate(g, shape_channel, shape_head):
    """Gate kind from the shape of g: one log-decay per key channel or one per head."""
    if tuple(g.shape) == tuple(shape_head):
        return _lib.KDA_GATE_HEAD
    _check(g, "g", torch.float32, shape_channel)
    return _lib.KDA_GATE_CHANNEL


_PLAIN_OPTIONS = {}  # gate kind -> options with nothing else set (kept alive for byref)


def _options(gate, every=0, snapshots=None, snapshot_cu=None, gate_scale=None):
    """kda_options; gate_scale given = fused prologue (raw q, k, beta logits, raw gate inputs)."""
    if every == 0 and snapshots is None and snapshot_cu is None and gate_scale is None:
        opts = _PLAIN_OPTIONS.get(gate)
        if opts is None:
            opts = _PLAIN_OPTIONS[gate] = _lib.Options(gate, 0, None, None, 0, 0.0)
        return ctypes.byref(opts)
    return ctypes.byref(_lib.Options(gate, every, _ptr(snapshots), _ptr(snapshot_cu), int(gate_scale is not None),
                                     float(gate_scale or 0.0)))


def _workspace(nbytes, device, workspace):
    """The caller's workspace (a contiguous uint8 tensor on `device`) when it is large enough,
    else a new one."""
    if nbytes == 0:
        return None
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8, None, device)
        if workspace.numel() >= nbytes:
            return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def prefill_chunked(q, k, v, g, beta, state=None, *, chunk=64, out=None, state_out=None, final_state=True,
                    workspace=None, snapshot_every=0, snapshots=None, prologue_gate_scale=None):
    """Chunked prefill of B equal-length sequences.

    q, k [B,T,H,dk], v [B,T,H,dv] (float32 or bfloat16), g float32 log alpha, either
    [B,T,H,dk] (one decay per key channel, KDA) or [B,T,H] (one per head, Gated DeltaNet),
    beta [B,T,H] (same dtype as q), state [B,H,dk,dv] float32 or None.
    Returns (o [B,T,H,dv] float32, S_T [B,H,dk,dv] float32 or None), plus the state snapshots
    [B, T // (snapshot_every * chunk), H, dk, dv] when snapshot_every > 0 (the state after
    every snapshot_every chunks).

    prologue_gate_scale = s (not None): fused input prologue; q, k are raw (normalised inside),
    beta holds logits and g the raw gate inputs a (g = -s * softplus(a))."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    dev = q.device
    _check(q, "q", dt, (B, T, H, dk), dev)
    _check(k, "k", dt, (B, T, H, dk), dev)
    _check(v, "v", dt, (B, T, H, dv), dev)
    gate = _gate(g, (B, T, H, dk), (B, T, H))
    _check(g, "g", torch.float32, None, dev)
    _check(beta, "beta", dt, (B, T, H), dev)
    _check(state, "state", torch.float32, (B, H, dk, dv), dev)
    if snapshot_every > 0:
        shape = (B, T // (snapshot_every * chunk), H, dk, dv)
        if snapshots is None:
            snapshots = torch.empty(shape, dtype=torch.float32, device=dev)
        _check(snapshots, "snapshots", torch.float32, shape, dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    _check(out, "out", torch.float32, (B, T, H, dv), dev)
    if state_out is None and final_state:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _check(state_out, "state_out", torch.float32, (B, H, dk, dv), dev)
    ws_bytes = workspace_size(_lib.KDA_OP_PREFILL, B, T, H, dk, dv, dt, chunk)
    ws = _workspace(ws_bytes, dev, workspace)
    L = _lib.load()
    _lib.check(L.kda_prefill_chunked_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(out),
                                        _ptr(state_out), B, T, H, dk, dv, _DT[dt], chunk, _ptr(ws), ws_bytes,
                                        _options(gate, snapshot_every, snapshots, None, prologue_gate_scale),
                                        _stream(dev)))
    return (out, state_out, snapshots) if snapshot_every > 0 else (out, state_out)


def append_prefill(q, k, v, g, beta, cu_seqlens, state=None, *, chunk=64, out=None, state_out=None,
                   final_state=True, workspace=None, snapshot_every=0, snapshots=None, prologue_gate_scale=None,
                   no_alloc=False):
    """Append-prefill of N packed segments (token-major [T_total, H, d]) on carried states.

    cu_seqlens: int32 GPU tensor [N+1] (0, ..., T_total).  g [T_total,H,dk] or [T_total,H] (one
    decay per head).  state [N,H,dk,dv] float32 or None.
    Returns (o [T_total,H,dv] float32, S_T [N,H,dk,dv] float32 or None), plus, when
    snapshot_every > 0, (snapshots [R,H,dk,dv], snapshot_cu int32 [N+1]): the state after every
    snapshot_every chunks of each segment, segment n at rows snapshot_cu[n] .. snapshot_cu[n+1]-1.
    snapshot_cu is computed on the device (no host synchronisation), so the row count is not
    known here: snapshots (given, or allocated) has R = T_total // (snapshot_every * chunk) rows,
    an upper bound of snapshot_cu[N]; rows from snapshot_cu[N] on are not written.

    no_alloc=True calls kda_append_prefill_noalloc: the library's fixed device scratch replaces
    the workspace (no workspace argument; calls needing more than KDA_NOALLOC_SCRATCH_BYTES of
    scratch raise).  Outputs not given are still allocated here."""
    T, H, dk = q.shape
    dv = v.shape[-1]
    N = cu_seqlens.numel() - 1
    dt = q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    dev = q.device
    _check(q, "q", dt, (T, H, dk), dev)
    _check(k, "k", dt, (T, H, dk), dev)
    _check(v, "v", dt, (T, H, dv), dev)
    gate = _gate(g, (T, H, dk), (T, H))
    _check(g, "g", torch.float32, None, dev)
    _check(beta, "beta", dt, (T, H), dev)
    _check(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    _check(state, "state", torch.float32, (N, H, dk, dv), dev)
    snapshot_cu = None
    if snapshot_every > 0:
        # per-segment snapshot counts from the segment lengths, on the device
        counts = torch.diff(cu_seqlens.to(torch.int64)) // (snapshot_every * chunk)
        snapshot_cu = torch.zeros(N + 1, dtype=torch.int32, device=dev)
        snapshot_cu[1:] = torch.cumsum(counts, 0).to(torch.int32)
        rows = T // (snapshot_every * chunk)
        if snapshots is None:
            snapshots = torch.empty((rows, H, dk, dv), dtype=torch.float32, device=dev)
        _check(snapshots, "snapshots", torch.float32, None, dev)
        if snapshots.dim() != 4 or tuple(snapshots.shape[1:]) != (H, dk, dv) or snapshots.shape[0] < rows:
            raise ValueError(f"snapshots must be [>= {rows}, {H}, {dk}, {dv}], got {tuple(snapshots.shape)}")
    elif snapshots is not None:
        raise ValueError("snapshots given without snapshot_every")
    if out is None:
        out = torch.empty((T, H, dv), dtype=torch.float32, device=dev)
    _check(out, "out", torch.float32, (T, H, dv), dev)
    if state_out is None and final_state:
        state_out = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    _check(state_out, "state_out", torch.float32, (N, H, dk, dv), dev)
    L = _lib.load()
    opts = _options(gate, snapshot_every, snapshots, snapshot_cu, prologue_gate_scale)
    if no_alloc:
        if workspace is not None:
            raise ValueError("no_alloc takes no workspace")
        _lib.check(L.kda_append_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, T,
                                                _ptr(state), _ptr(out), _ptr(state_out), H, dk, dv, _DT[dt], chunk,
                                                opts, _stream(dev)))
        if snapshot_every > 0:
            return out, state_out, snapshots, snapshot_cu
        return out, state_out
    ws_bytes = workspace_size(_lib.KDA_OP_APPEND, N, T, H, dk, dv, dt, chunk)
    ws = _workspace(ws_bytes, dev, workspace)
    _lib.check(L.kda_append_prefill_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, T,
                                       _ptr(state), _ptr(out), _ptr(state_out), H, dk, dv, _DT[dt], chunk,
                                       _ptr(ws), ws_bytes, opts, _stream(dev)))
    if snapshot_every > 0:
        return out, state_out, snapshots, snapshot_cu
    return out, state_out


def chunked_backward(q, k, v, g, beta, cu_seqlens, state=None, *, d_out, d_state_out=None, chunk=64,
                     state_grad=True, workspace=None):
    """Gradients of ``append_prefill`` (packed segments, token-major [T_total, H, d]).

    d_out [T_total,H,dv] float32 = dL/do; d_state_out [N,H,dk,dv] float32 = dL/dS_T or None (zero).
    Returns (dq, dk [T_total,H,dk], dv [T_total,H,dv], dg (g's shape), dbeta [T_total,H],
    dS0 [N,H,dk,dv] or None when state_grad is False), all float32.  A batch of B equal
    sequences of T tokens is the packed layout [B*T, H, d] with cu_seqlens = 0, T, ..., B*T."""
    T, H, dk = q.shape
    dv = v.shape[-1]
    N = cu_seqlens.numel() - 1
    dt = q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    dev = q.device
    _check(q, "q", dt, (T, H, dk), dev)
    _check(k, "k", dt, (T, H, dk), dev)
    _check(v, "v", dt, (T, H, dv), dev)
    gate = _gate(g, (T, H, dk), (T, H))
    _check(g, "g", torch.float32, None, dev)
    _check(beta, "beta", dt, (T, H), dev)
    _check(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    _check(state, "state", torch.float32, (N, H, dk, dv), dev)
    _check(d_out, "d_out", torch.float32, (T, H, dv), dev)
    _check(d_state_out, "d_state_out", torch.float32, (N, H, dk, dv), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    dq, dk_, dv_ = torch.empty((T, H, dk), **f32), torch.empty((T, H, dk), **f32), torch.empty((T, H, dv), **f32)
    dg = torch.empty(tuple(g.shape), **f32)
    db = torch.empty((T, H), **f32)
    ds0 = torch.empty((N, H, dk, dv), **f32) if state_grad else None
    ws_bytes = workspace_size(_lib.KDA_OP_BACKWARD, N, T, H, dk, dv, dt, chunk)
    ws = _workspace(ws_bytes, dev, workspace)
    L = _lib.load()
    _lib.check(L.kda_chunked_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, T,
                                      _ptr(state), _ptr(d_out), _ptr(d_state_out), _ptr(dq), _ptr(dk_), _ptr(dv_),
                                      _ptr(dg), _ptr(db), _ptr(ds0), H, dk, dv, _DT[dt], chunk, _ptr(ws), ws_bytes,
                                      _options(gate), _stream(dev)))
    return dq, dk_, dv_, dg, db, ds0


def decode_step(q, k, v, g, beta, state, *, out=None, state_out=None, prologue_gate_scale=None):
    """One decode step for N sequences: q, k [N,H,dk], g [N,H,dk] or [N,H] (one decay per head),
    v [N,H,dv], beta [N,H], state [N,H,dk,dv].

    The state is updated in place unless ``state_out`` is given.  Returns o [N,H,dv] float32."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    dev = q.device
    _check(q, "q", dt, (N, H, dk), dev)
    _check(k, "k", dt, (N, H, dk), dev)
    _check(v, "v", dt, (N, H, dv), dev)
    gate = _gate(g, (N, H, dk), (N, H))
    _check(g, "g", torch.float32, None, dev)
    _check(beta, "beta", dt, (N, H), dev)
    _check(state, "state", torch.float32, (N, H, dk, dv), dev)
    if state_out is None:
        state_out = state
    _check(state_out, "state_out", torch.float32, (N, H, dk, dv), dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    _check(out, "out", torch.float32, (N, H, dv), dev)
    L = _lib.load()
    _lib.check(L.kda_decode_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                                    _ptr(state_out), _ptr(out), N, H, dk, dv, _DT[dt],
                                    _options(gate, gate_scale=prologue_gate_scale),
                                    _stream(dev)))
    return out
