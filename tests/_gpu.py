"""Helpers for GPU tests: upload synthetic tensors, download results (test infrastructure)."""
import numpy as np
import torch

import synth


def dev(x: np.ndarray, dtype: str, device="cuda"):
    """Upload a stored tensor (float32, or uint16 bfloat16 bits) to the GPU."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def f64(x, dtype):
    return synth.to_f64(x, dtype)


def make_inputs(w, T, offset_tokens=0, q_unit=None):
    """Stored tensors (numpy) + their fp64 widening for the oracle."""
    q, k, v, g, b = synth.gen_tokens(w, T, offset_tokens=offset_tokens, q_unit=q_unit)
    st = (q, k, v, g, b)
    wide = (f64(q, w.dtype), f64(k, w.dtype), f64(v, w.dtype), g.astype(np.float64), f64(b, w.dtype))
    return st, wide


def upload(w, st, batch_shape=None):
    q, k, v, g, b = st
    ts = [dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype), dev(g, "f32"), dev(b, w.dtype)]
    if batch_shape is not None:
        ts = [t.reshape(*batch_shape, *t.shape[1:]) for t in ts]
    return ts
