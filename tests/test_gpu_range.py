"""GPU parity where values leave the fp16 range of the bfloat16 path's matrix-core operands, and
the debug check of device-resident arguments.

The bfloat16 path rounds q, k, beta*v, the per-token corrections, the state and the chunk factors
to fp16 operands.  Every such value is checked against the fp16 range first, and a chain that
meets one outside it is recomputed by the fp32 chunked kernel in the same call.  The bar is the
bfloat16 tolerance (per sequence-head slice max|gpu - oracle| / max|oracle| <= 2e-3), whatever
the magnitudes.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_75_amd as kda
import oracle
import synth
from _gpu import dev, host, make_inputs, upload
from _util import assert_close

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL = 2e-3


def _w(seed, v_std=1.0, s0_std=0.02, H=3):
    return synth.Workload("range", seed, H=H, dk=128, dv=128, dtype="bf16", chunk=64, s0_std=s0_std, v_std=v_std)


@pytest.mark.parametrize("v_std,s0_std,in_place", [
    (2e4, 1e4, False),   # beta*v, the corrections and the state all leave the fp16 range
    (2e4, 1e4, True),    # the same with state_out = state_in
    (300.0, 100.0, False),  # large but inside the range: stays on the matrix cores
])
def test_magnitudes_match_oracle(v_std, s0_std, in_place):
    print(f"range v_std={v_std} s0_std={s0_std} in_place={in_place}", flush=True)
    w = _w(61, v_std, s0_std)
    B, T = 2, 333
    st, wide = make_inputs(w, B * T)
    s0 = synth.gen_state(w, B)
    q, k, v, g, b = upload(w, st, (B, T))
    S = dev(s0, "f32")
    if in_place:
        o, sT = kda.prefill_chunked(q, k, v, g, b, S, state_out=S)
    else:
        o, sT = kda.prefill_chunked(q, k, v, g, b, S)
    torch.cuda.synchronize()
    cu = np.arange(B + 1) * T
    oref, sref = oracle.recurrence(*wide, cu, s0)
    bv = np.abs(wide[2] * wide[4][..., None]).max()  # the largest beta*v the kernels stage in fp16
    assert (bv > 65504.0) if v_std > 1e4 else (bv < 65504.0 and np.abs(oref).max() > 1e2)
    assert_close(host(o).reshape(B * T, w.H, w.dv), oref, TOL, cu, "o")
    assert_close(host(sT), sref, TOL, None, "S_T")


def test_out_of_range_segments_next_to_normal_ones():
    """Packed segments: one with v scaled far beyond fp16, one with queries beyond the allowed
    entry size, two ordinary ones; in-place states.  Every segment matches the oracle, and the
    ordinary segments' outputs and states are bitwise those of a call in which no segment is out
    of range (the fp32 redo touches only the chains that need it)."""
    w = _w(67)
    lengths = [150, 200, 64, 99]
    cu = synth.cu_seqlens(lengths)
    T, N = int(cu[-1]), len(lengths)
    print(f"out-of-range segments lengths={lengths}", flush=True)
    st, wide = make_inputs(w, T)
    s0 = synth.gen_state(w, N)

    def scaled(x, f):  # bf16 bits scaled by a power of two: exact
        return (synth.bf16_bits_to_f32(x) * np.float32(f)).view(np.uint32).__rshift__(16).astype(np.uint16)

    q, k, v, g, b = (np.array(x) for x in st)
    v[cu[1]:cu[2]] = scaled(v[cu[1]:cu[2]], 2.0 ** 17)
    q[cu[2]:cu[3]] = scaled(q[cu[2]:cu[3]], 2.0 ** 18)
    wide2 = (synth.to_f64(q, "bf16"), wide[1], synth.to_f64(v, "bf16"), wide[3], wide[4])
    cu_d = torch.from_numpy(cu).cuda()
    ta = upload(w, st)
    tb = upload(w, (q, k, v, g, b))
    S_a, S_b = dev(s0, "f32"), dev(s0, "f32")
    oa, sa = kda.append_prefill(*ta, cu_d, S_a, state_out=S_a)
    ob, sb = kda.append_prefill(*tb, cu_d, S_b, state_out=S_b)
    torch.cuda.synchronize()
    oref, sref = oracle.recurrence(*wide2, cu, s0)
    assert_close(host(ob), oref, TOL, cu, "o")
    assert_close(host(sb), sref, TOL, None, "S_T")
    for n in (0, 3):
        assert torch.equal(ob[cu[n]:cu[n + 1]], oa[cu[n]:cu[n + 1]])
        assert torch.equal(sb[n], sa[n])


def test_debug_check_rejects_bad_device_arguments(monkeypatch):
    """KDA_DEBUG_CHECK=1: the call copies cu_seqlens and the gates to the host and returns
    KDA_ERR_INVALID_ARG before any launch (outputs untouched).  The malformed offsets used here
    stay inside the buffers, so they could do no harm even if they were launched."""
    monkeypatch.setenv("KDA_DEBUG_CHECK", "1")
    w = _w(71, H=2)
    T = 100
    st, wide = make_inputs(w, T)
    q, k, v, g, b = upload(w, st)
    canary = 777.0
    out = torch.full((T, w.H, w.dv), canary, device="cuda")
    # a well-formed call passes the check and computes as usual
    good = torch.tensor([0, 40, 100], dtype=torch.int32, device="cuda")
    o, s = kda.append_prefill(q, k, v, g, b, good, out=out)
    torch.cuda.synchronize()
    oref, _ = oracle.recurrence(*wide, np.array([0, 40, 100]))
    assert_close(host(o), oref, TOL, np.array([0, 40, 100]), "o")
    bad = [([0, 40, 20, 100], b"decreases"), ([0, 50, 90], b"T_total"), ([5, 50, 100], b"[0]")]
    for cu, msg in bad:
        out.fill_(canary)
        with pytest.raises(kda.KdaError) as ei:
            kda.append_prefill(q, k, v, g, b, torch.tensor(cu, dtype=torch.int32, device="cuda"), out=out)
        assert ei.value.status == -1 and msg.decode() in str(ei.value)
        torch.cuda.synchronize()
        assert torch.all(out == canary)
    gpos = g.clone()
    gpos[7, 1, 3] = 0.5  # a log-decay above 0 (alpha > 1)
    with pytest.raises(kda.KdaError, match="g\\["):
        kda.prefill_chunked(q[None], k[None], v[None], gpos[None], b[None], out=out[None])
    bbig = b.clone()
    bbig[3, 0] = 1.5
    with pytest.raises(kda.KdaError, match="beta"):
        kda.decode_step(q[:1], k[:1], v[:1], g[:1], bbig[3:4], torch.zeros((1, w.H, 128, 128), device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(out == canary)
