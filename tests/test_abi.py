"""C-ABI contract on the host: the library loads and exports every symbol include/kda.h declares;
argument validation rejects bad calls before any device work (no GPU needed: every call here
fails validation, so nothing is launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from gated_delta_rule_75_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("HIP library not built")
    return _lib, _lib.load()


def test_exports_match_header():
    _l, L = _lib()
    header = open(os.path.join(ROOT, "include", "kda.h")).read()
    declared = set(re.findall(r"\b(kda_[a-z_]+)\s*\(", header))
    assert declared == set(_l.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings_and_version():
    _l, L = _lib()
    assert L.kda_version().decode().startswith("kda-mi355x")
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert L.kda_status_string(s)
    assert L.kda_status_string(-99) == b"unknown status"


def test_supported_and_workspace():
    _l, L = _lib()
    assert L.kda_is_supported(0, 1, 128, 128, 64) == 1
    assert L.kda_is_supported(0, 0, 16, 16, 16) == 1
    assert L.kda_is_supported(0, 1, 96, 128, 64) == 0
    assert L.kda_is_supported(2, 1, 128, 128, 0) == 1
    assert L.kda_workspace_size(2, 4, 0, 32, 128, 128, 1, 64) == 0
    ws = L.kda_workspace_size(0, 1, 8192, 32, 128, 128, 1, 64)
    assert ws == 128 * 32 * 61952 + 128 * 32 * 4  # records, then one flag word per record
    assert L.kda_workspace_size(0, 1, 8192, 32, 96, 128, 1, 64) == 2 ** 64 - 1


FAKE = 0x100000  # 16-byte aligned, never dereferenced: validation fails first


def test_validation_errors_launch_nothing():
    _l, L = _lib()
    P = FAKE
    # unsupported head size
    rc = L.kda_prefill_chunked(P, P, P, P, P, None, P, None, 1, 64, 2, 96, 128, 1, 64, None, 0, None)
    assert rc == _l.KDA_ERR_UNSUPPORTED and b"d_k=96" in L.kda_last_error()
    # negative sizes / bad dtype
    assert L.kda_prefill_chunked(P, P, P, P, P, None, P, None, -1, 64, 2, 16, 16, 0, 16, None, 0, None) == -1
    assert L.kda_prefill_chunked(P, P, P, P, P, None, P, None, 1, 64, 2, 16, 16, 7, 16, None, 0, None) == -1
    # missing inputs
    assert L.kda_prefill_chunked(None, P, P, P, P, None, P, None, 1, 64, 2, 16, 16, 0, 16, None, 0, None) == -1
    # a chunk's rows must fit 32-bit byte offsets: H * max(d_k, d_v) below 2^23
    rc = L.kda_prefill_chunked(P, P, P, P, P, None, P, None, 1, 64, 1 << 16, 128, 128, 1, 64, None, 0, None)
    assert rc == _l.KDA_ERR_INVALID_ARG and b"2^23" in L.kda_last_error()
    S = 1 << 41
    rc = L.kda_decode_step(P, P + 4096, P + 8192, P + 12288, P + 16384, S, S, 1 << 42, 1, 1 << 19, 16, 16, 0, None)
    assert rc == _l.KDA_ERR_INVALID_ARG and b"2^23" in L.kda_last_error()
    # misaligned (q must be 16-byte aligned for prefill; decode states too)
    assert L.kda_prefill_chunked(P + 4, P, P, P, P, None, P, None, 1, 64, 2, 16, 16, 0, 16, None, 0, None) == -3
    assert L.kda_decode_step(P, P, P, P, P, 1 << 41, (1 << 41) + 4, 1 << 42, 1, 1, 16, 16, 0, None) == -3
    # workspace too small for the matrix-core path
    big = 1 << 40
    rc = L.kda_prefill_chunked(P, P, P, P, P, None, big, None, 1, 64, 2, 128, 128, 1, 64, None, 0, None)
    assert rc == _l.KDA_ERR_WORKSPACE
    # output overlapping an input
    rc = L.kda_prefill_chunked(P, P, P, P, P, None, P, None, 1, 64, 2, 16, 16, 0, 16, None, 0, None)
    assert rc == _l.KDA_ERR_ALIAS
    # state_out partially overlapping state_in (decode)
    S = 1 << 41
    rc = L.kda_decode_step(P, P + 4096, P + 8192, P + 12288, P + 16384, S, S + 16, 1 << 42, 1, 1, 16, 16, 0, None)
    assert rc == _l.KDA_ERR_ALIAS
    # decode without a state
    assert L.kda_decode_step(P, P, P, P, P, None, None, P, 1, 1, 16, 16, 0, None) == -1
    # append without cu_seqlens
    assert L.kda_append_prefill(P, P, P, P, P, None, 1, 10, None, P, None, 2, 16, 16, 0, 16, None, 0, None) == -1


def test_injected_launch_failure_reports_hip_error(monkeypatch):
    _l, L = _lib()
    monkeypatch.setenv("KDA_TEST_FAIL_LAUNCH", "1")
    # valid, non-overlapping fake buffers: validation passes, then the injected failure returns
    # before anything touches the device
    base = 1 << 40
    ptrs = [base + i * (1 << 30) for i in range(8)]
    rc = L.kda_decode_step(*ptrs[:5], ptrs[5], ptrs[5], ptrs[6], 1, 1, 16, 16, 0, None)
    assert rc == _l.KDA_ERR_HIP and b"injected" in L.kda_last_error()


def test_extended_call_options_are_validated():
    """Options of the extended calls: gate kind, snapshot spacing and buffers (host-side checks,
    nothing is launched)."""
    import ctypes

    _l, L = _lib()
    base = 1 << 40
    p = [base + i * (1 << 30) for i in range(12)]  # valid, non-overlapping fake buffers

    def opts(gate=0, every=0, snaps=None, snap_cu=None, prologue=0, scale=0.0):
        return ctypes.byref(_l.Options(gate, every, snaps, snap_cu, prologue, scale))

    def prefill(o):
        return L.kda_prefill_chunked_ex(p[0], p[1], p[2], p[3], p[4], None, p[5], None, 1, 64, 2, 16, 16, 0, 16,
                                        None, 0, o, None)

    def append(o):
        return L.kda_append_prefill_ex(p[0], p[1], p[2], p[3], p[4], p[6], 1, 64, None, p[5], None, 2, 16, 16, 0,
                                       16, None, 0, o, None)

    def decode(o):
        return L.kda_decode_step_ex(p[0], p[1], p[2], p[3], p[4], p[7], p[7], p[5], 1, 1, 16, 16, 0, o, None)

    assert prefill(opts(gate=2)) == _l.KDA_ERR_INVALID_ARG and b"gate" in L.kda_last_error()
    assert prefill(opts(prologue=2)) == _l.KDA_ERR_INVALID_ARG and b"prologue" in L.kda_last_error()
    assert prefill(opts(prologue=1, scale=0.0)) == _l.KDA_ERR_INVALID_ARG and b"gate_scale" in L.kda_last_error()
    assert decode(opts(prologue=1, scale=float("inf"))) == _l.KDA_ERR_INVALID_ARG
    assert prefill(opts(every=-1)) == _l.KDA_ERR_INVALID_ARG
    assert prefill(opts(every=1)) == _l.KDA_ERR_INVALID_ARG and b"snapshots" in L.kda_last_error()
    assert prefill(opts(every=1, snaps=p[8] + 2)) == _l.KDA_ERR_MISALIGNED
    assert prefill(opts(every=1, snaps=p[0])) == _l.KDA_ERR_ALIAS  # snapshots on top of q
    assert append(opts(every=1, snaps=p[8])) == _l.KDA_ERR_INVALID_ARG and b"snapshot_cu" in L.kda_last_error()
    assert append(opts(every=1, snaps=p[6], snap_cu=p[9])) == _l.KDA_ERR_ALIAS  # snapshots on cu_seqlens
    assert decode(opts(every=1, snaps=p[8])) == _l.KDA_ERR_INVALID_ARG and b"snapshot" in L.kda_last_error()
    # per-head gate: g is [T, H] (4-byte alignment suffices), channel gate: 16 bytes for prefill
    assert L.kda_prefill_chunked_ex(p[0], p[1], p[2], p[3] + 4, p[4], None, p[5], None, 1, 64, 2, 16, 16, 0, 16,
                                    None, 0, opts(gate=0), None) == _l.KDA_ERR_MISALIGNED


def test_python_options_marshalling():
    """The binding's option struct matches struct kda_options field for field."""
    import ctypes

    import gated_delta_rule_75_amd as kda
    from gated_delta_rule_75_amd import _lib as _l

    o = _l.Options(_l.KDA_GATE_HEAD, 3, 0x1000, 0x2000, 1, 0.5)
    assert (o.gate, o.snapshot_every, o.snapshots, o.snapshot_cu, o.prologue, o.gate_scale) == (1, 3, 0x1000, 0x2000,
                                                                                                   1, 0.5)
    assert ctypes.sizeof(o) == 32  # int32, int32, pointer, pointer, int32, float
    assert kda._options(_l.KDA_GATE_CHANNEL) is not None


def test_backward_call_is_validated():
    """kda_chunked_backward: shapes, required buffers, options, aliasing and workspace are checked
    on the host before anything is launched."""
    import ctypes

    _l, L = _lib()
    base = 1 << 40
    p = [base + i * (1 << 30) for i in range(20)]  # valid, non-overlapping fake buffers
    N, T, H, d, C = 1, 64, 2, 16, 16
    need = L.kda_workspace_size(_l.KDA_OP_BACKWARD, N, T, H, d, d, 0, C)
    assert 0 < need < (1 << 40) and L.kda_is_supported(_l.KDA_OP_BACKWARD, 0, d, d, C) == 1
    assert L.kda_is_supported(_l.KDA_OP_BACKWARD, 1, 128, 64, 64) == 0  # d_k != d_v

    def call(**kw):
        a = dict(q=p[0], k=p[1], v=p[2], g=p[3], beta=p[4], cu=p[5], s0=None, d_out=p[6], dsT=None, dq=p[7],
                 dk=p[8], dv=p[9], dg=p[10], db=p[11], ds0=None, d_k=d, d_v=d, chunk=C, ws=p[12], ws_bytes=need,
                 opts=None)
        a.update(kw)
        return L.kda_chunked_backward(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], N, T, a["s0"], a["d_out"],
                                      a["dsT"], a["dq"], a["dk"], a["dv"], a["dg"], a["db"], a["ds0"], H, a["d_k"],
                                      a["d_v"], 0, a["chunk"], a["ws"], a["ws_bytes"], a["opts"], None)

    assert call(d_v=32) == _l.KDA_ERR_UNSUPPORTED
    assert call(chunk=128) == _l.KDA_ERR_UNSUPPORTED
    assert call(d_out=None) == _l.KDA_ERR_INVALID_ARG and b"d_out" in L.kda_last_error()
    assert call(cu=None) == _l.KDA_ERR_INVALID_ARG
    assert call(dq=p[0]) == _l.KDA_ERR_ALIAS  # a gradient on top of q
    assert call(dk=p[7]) == _l.KDA_ERR_ALIAS  # two gradients on one buffer
    assert call(ws=p[6]) == _l.KDA_ERR_ALIAS  # workspace on top of d_out
    assert call(ws_bytes=need - 1) == _l.KDA_ERR_WORKSPACE
    assert call(ws=None) == _l.KDA_ERR_WORKSPACE
    assert call(dg=p[10] + 2) == _l.KDA_ERR_MISALIGNED
    snap = ctypes.byref(_l.Options(0, 1, p[13], p[14], 0, 0.0))
    assert call(opts=snap) == _l.KDA_ERR_UNSUPPORTED and b"snapshots" in L.kda_last_error()
    pro = ctypes.byref(_l.Options(0, 0, None, None, 1, 1.0))
    assert call(opts=pro) == _l.KDA_ERR_UNSUPPORTED


def test_workspace_may_not_overlap_arguments():
    """Prefill and append reject a workspace that overlaps an input or an output (the prep pass
    writes its records while other workgroups still read the inputs)."""
    _l, L = _lib()
    base = 1 << 40
    p = [base + i * (1 << 30) for i in range(12)]  # valid, non-overlapping fake buffers
    B, T, H, d, C = 1, 64, 2, 128, 64
    need = L.kda_workspace_size(_l.KDA_OP_PREFILL, B, T, H, d, d, _l.KDA_BF16, C)
    need_a = L.kda_workspace_size(_l.KDA_OP_APPEND, 1, T, H, d, d, _l.KDA_BF16, C)
    assert need > 0 and need_a > 0

    def prefill(ws, s_in=None, s_out=None):
        return L.kda_prefill_chunked(p[0], p[1], p[2], p[3], p[4], s_in, p[5], s_out, B, T, H, d, d, _l.KDA_BF16, C,
                                     ws, need, None)

    def append(ws, s_in=None, s_out=None):
        return L.kda_append_prefill(p[0], p[1], p[2], p[3], p[4], p[6], 1, T, s_in, p[5], s_out, H, d, d,
                                    _l.KDA_BF16, C, ws, need_a, None)

    for call in (prefill, append):
        assert call(p[0]) == _l.KDA_ERR_ALIAS and b"workspace" in L.kda_last_error()  # on q
        assert call(p[3] + 256) == _l.KDA_ERR_ALIAS  # inside g
        assert call(p[5]) == _l.KDA_ERR_ALIAS  # on out
        assert call(p[8], s_in=p[7], s_out=p[8]) == _l.KDA_ERR_ALIAS  # on state_out
        assert call(p[7], s_in=p[7]) == _l.KDA_ERR_ALIAS  # on state_in
    assert append(p[6]) == _l.KDA_ERR_ALIAS  # on cu_seqlens
    assert prefill(p[0] - need + 256) == _l.KDA_ERR_ALIAS  # ends inside q


def test_host_validators_reject_malformed_offsets_and_gates():
    """kda_validate_*: the checks KDA_DEBUG_CHECK=1 applies to device-resident data, on host arrays."""
    import numpy as np

    _l, L = _lib()

    def cu_ok(cu, T):
        a = np.ascontiguousarray(cu, dtype=np.int32)
        return L.kda_validate_cu_seqlens(a.ctypes.data, len(a) - 1, T)

    assert cu_ok([0, 5, 5, 12], 12) == 0
    assert cu_ok([0], 0) == 0
    assert cu_ok([1, 5, 12], 12) == _l.KDA_ERR_INVALID_ARG and b"[0]" in L.kda_last_error()
    assert cu_ok([0, 7, 5, 12], 12) == _l.KDA_ERR_INVALID_ARG and b"decreases" in L.kda_last_error()
    assert cu_ok([0, 5, 11], 12) == _l.KDA_ERR_INVALID_ARG and b"T_total" in L.kda_last_error()
    assert cu_ok([0, 5, 13], 12) == _l.KDA_ERR_INVALID_ARG
    assert L.kda_validate_cu_seqlens(None, 1, 0) == _l.KDA_ERR_INVALID_ARG

    def snap_ok(cu, scu, every, chunk):
        a = np.ascontiguousarray(cu, dtype=np.int32)
        b = np.ascontiguousarray(scu, dtype=np.int32)
        return L.kda_validate_snapshot_cu(a.ctypes.data, b.ctypes.data, len(a) - 1, every, chunk)

    cu = [0, 200, 200, 263]  # lengths 200, 0, 63 with snapshots every 64 tokens: 3, 0, 0
    assert snap_ok(cu, [0, 3, 3, 3], 1, 64) == 0
    assert snap_ok(cu, [0, 3, 3, 4], 1, 64) == _l.KDA_ERR_INVALID_ARG
    assert snap_ok(cu, [1, 4, 4, 4], 1, 64) == _l.KDA_ERR_INVALID_ARG
    assert snap_ok(cu, [0, 1, 1, 1], 2, 64) == 0  # every 128 tokens: 1, 0, 0

    def gates_ok(g, b, raw=0):
        ga = np.ascontiguousarray(g, dtype=np.float32)
        ba = np.ascontiguousarray(b, dtype=np.float32)
        return L.kda_validate_gates(ga.ctypes.data, ga.size, ba.ctypes.data, ba.size, raw)

    assert gates_ok([0.0, -0.1, -30.0], [0.0, 0.5, 1.0]) == 0
    assert gates_ok([0.0, 0.25], [0.5]) == _l.KDA_ERR_INVALID_ARG and b"g[1]" in L.kda_last_error()
    assert gates_ok([-np.inf], [0.5]) == _l.KDA_ERR_INVALID_ARG
    assert gates_ok([np.nan], [0.5]) == _l.KDA_ERR_INVALID_ARG
    assert gates_ok([-1.0], [1.5]) == _l.KDA_ERR_INVALID_ARG and b"beta[0]" in L.kda_last_error()
    assert gates_ok([-1.0], [-0.01]) == _l.KDA_ERR_INVALID_ARG
    assert gates_ok([2.0, -3.0], [-4.0, 7.0], raw=1) == 0  # raw prologue inputs: any finite value
    assert gates_ok([np.inf], [0.0], raw=1) == _l.KDA_ERR_INVALID_ARG


def test_binding_rejects_a_host_workspace():
    """The binding checks a caller's workspace like every other tensor before passing its pointer."""
    import torch

    import gated_delta_rule_75_amd as kda

    with pytest.raises(ValueError, match="GPU tensor"):
        kda._workspace(1024, torch.device("cuda:0"), torch.empty(4096, dtype=torch.uint8))
