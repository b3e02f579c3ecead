"""ctypes loader of the in-tree HIP library ``_kda.so`` (declarations: include/kda.h).

The library is loaded after ``import torch`` so that it binds to the HIP runtime torch
already loaded (one runtime per process).  A missing library is an error: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime first)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_kda.so")

KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_MISALIGNED = 0, -1, -2, -3
KDA_ERR_ALIAS, KDA_ERR_WORKSPACE, KDA_ERR_HIP = -4, -5, -6
KDA_F32, KDA_BF16 = 0, 1
KDA_OP_PREFILL, KDA_OP_APPEND, KDA_OP_DECODE, KDA_OP_BACKWARD = 0, 1, 2, 3
KDA_GATE_CHANNEL, KDA_GATE_HEAD = 0, 1
KDA_NOALLOC_SCRATCH_BYTES = 128 << 20  # the fixed device scratch of kda_append_prefill_noalloc

# every symbol include/kda.h declares
EXPORTS = ("kda_prefill_chunked", "kda_append_prefill", "kda_decode_step", "kda_prefill_chunked_ex",
           "kda_append_prefill_ex", "kda_decode_step_ex", "kda_append_prefill_noalloc", "kda_chunked_backward", "kda_workspace_size",
           "kda_is_supported", "kda_validate_cu_seqlens", "kda_validate_snapshot_cu", "kda_validate_gates",
           "kda_status_string", "kda_last_error", "kda_version", "kda_timing_begin", "kda_timing_end")
KERNEL_NAMES = {1: "kda_prep", 2: "kda_state", 3: "kda_chunk_f32", 4: "kda_decode", 5: "kda_bwd_factors",
                6: "kda_bwd_fwd_chain", 7: "kda_bwd_rev_chain", 8: "kda_bwd_grad_state", 9: "kda_bwd_grad_chunk"}

_LIB = None


class Options(ctypes.Structure):
    """struct kda_options"""
    _fields_ = [("gate", ctypes.c_int32), ("snapshot_every", ctypes.c_int32), ("snapshots", ctypes.c_void_p),
                ("snapshot_cu", ctypes.c_void_p), ("prologue", ctypes.c_int32), ("gate_scale", ctypes.c_float)]


class KdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def load():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"KDA HIP library not built: {LIB_PATH} (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.kda_prefill_chunked.restype = ctypes.c_int
    L.kda_prefill_chunked.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, i32, vp, sz, vp]
    L.kda_append_prefill.restype = ctypes.c_int
    L.kda_append_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, vp, vp, vp, i32, i32, i32, i32, i32, vp, sz,
                                     vp]
    L.kda_decode_step.restype = ctypes.c_int
    L.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    op = ctypes.POINTER(Options)
    L.kda_prefill_chunked_ex.restype = ctypes.c_int
    L.kda_prefill_chunked_ex.argtypes = L.kda_prefill_chunked.argtypes[:-1] + [op, vp]
    L.kda_append_prefill_ex.restype = ctypes.c_int
    L.kda_append_prefill_ex.argtypes = L.kda_append_prefill.argtypes[:-1] + [op, vp]
    L.kda_decode_step_ex.restype = ctypes.c_int
    L.kda_decode_step_ex.argtypes = L.kda_decode_step.argtypes[:-1] + [op, vp]
    L.kda_append_prefill_noalloc.restype = ctypes.c_int
    L.kda_append_prefill_noalloc.argtypes = L.kda_append_prefill.argtypes[:-3] + [op, vp]
    L.kda_workspace_size.restype = sz
    L.kda_chunked_backward.restype = ctypes.c_int
    L.kda_chunked_backward.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32,
                                       i32, i32, i32, vp, sz, op, vp]
    L.kda_workspace_size.argtypes = [i32, i64, i64, i32, i32, i32, i32, i32]
    L.kda_is_supported.restype = ctypes.c_int
    L.kda_is_supported.argtypes = [i32, i32, i32, i32, i32]
    L.kda_status_string.restype = ctypes.c_char_p
    L.kda_status_string.argtypes = [ctypes.c_int]
    L.kda_last_error.restype = ctypes.c_char_p
    L.kda_last_error.argtypes = []
    L.kda_version.restype = ctypes.c_char_p
    L.kda_version.argtypes = []
    L.kda_timing_begin.restype = ctypes.c_int
    L.kda_timing_begin.argtypes = []
    L.kda_timing_end.restype = ctypes.c_int
    L.kda_timing_end.argtypes = [vp, vp, i32]
    L.kda_validate_cu_seqlens.restype = ctypes.c_int
    L.kda_validate_cu_seqlens.argtypes = [vp, i32, i64]
    L.kda_validate_snapshot_cu.restype = ctypes.c_int
    L.kda_validate_snapshot_cu.argtypes = [vp, vp, i32, i32, i32]
    L.kda_validate_gates.restype = ctypes.c_int
    L.kda_validate_gates.argtypes = [vp, i64, vp, i64, i32]
    _LIB = L
    return L


def check(status: int):
    if status != KDA_OK:
        L = load()
        msg = L.kda_last_error().decode() or L.kda_status_string(status).decode()
        raise KdaError(status, msg)
