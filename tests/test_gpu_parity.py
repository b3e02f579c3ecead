"""GPU parity of the HIP path against the fp64 oracle (small and medium sizes, edge cases).

Tolerance (per sequence-head slice, max|gpu - oracle| / max|oracle|): 2e-3 for bfloat16
storage (fp16 matrix-core operands, fp32 state), 1e-5 for fp32 storage (fp32 arithmetic).
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

TOL = {"bf16": 2e-3, "f32": 1e-5}


def _w(dtype="bf16", H=4, d=128, chunk=64, seed=1, s0_std=0.0, gate=None):
    w = synth.Workload("t", seed, H=H, dk=d, dv=d, dtype=dtype, chunk=chunk, s0_std=s0_std)
    if gate is not None:
        w.gate = gate
    return w


def _run_prefill(w, B, T, with_state):
    st, wide = make_inputs(w, B * T)
    s0 = synth.gen_state(w, B) if with_state else None
    q, k, v, g, b = upload(w, st, (B, T))
    S0 = dev(s0, "f32") if s0 is not None else None
    o, sT = kda.prefill_chunked(q, k, v, g, b, S0, chunk=w.chunk)
    torch.cuda.synchronize()
    cu = np.arange(B + 1) * T
    oref, sref = oracle.recurrence(*wide, cu, s0)
    return host(o).reshape(B * T, w.H, w.dv), host(sT), oref, sref, cu


@pytest.mark.parametrize("dtype,d,chunk,B,T,with_state", [
    ("f32", 16, 16, 1, 64, False),      # the tiny fp32 workload's shape
    ("f32", 16, 16, 2, 37, True),
    ("f32", 32, 32, 1, 100, True),
    ("f32", 64, 16, 1, 70, False),
    ("f32", 128, 32, 1, 70, True),
    ("bf16", 64, 32, 2, 50, True),      # bf16 storage through the fp32 kernel
    ("bf16", 128, 64, 1, 64, False),    # one full chunk
    ("bf16", 128, 64, 1, 128, True),    # two chunks: one pass of the two-chunk loop
    ("bf16", 128, 64, 1, 130, True),    # three chunks, the last two tokens long
    ("bf16", 128, 64, 1, 1000, False),  # several chunks + ragged tail
    ("bf16", 128, 64, 2, 333, True),
    ("bf16", 128, 64, 1, 1, True),      # a single token
    ("bf16", 128, 64, 1, 0, True),      # empty: state passes through
    ("bf16", 128, 64, 1, 4097, True),   # 65 chunks, the last one token long
    ("bf16", 128, 64, 2, 8292, True),   # two long sequences, ragged tail
])
def test_prefill_matches_oracle(dtype, d, chunk, B, T, with_state):
    print(f"prefill dtype={dtype} d={d} chunk={chunk} B={B} T={T} state={with_state}", flush=True)
    w = _w(dtype, H=3, d=d, chunk=chunk, seed=11 + T, s0_std=0.02 if with_state else 0.0)
    o, s, oref, sref, cu = _run_prefill(w, B, T, with_state)
    if T > 0:
        assert_close(o, oref, TOL[dtype], cu, "o")
    assert_close(s, sref, TOL[dtype], None, "S_T")


def test_prefill_in_place_state_and_no_final_state():
    """In-place state (state_out is state_in) and a call without a final state."""
    w = _w("bf16", H=2, d=128, chunk=64, seed=41, s0_std=0.02)
    B, T = 1, 64 * 64 + 64 * 3 + 5
    print(f"prefill in place B={B} T={T}", flush=True)
    st, wide = make_inputs(w, B * T)
    s0 = synth.gen_state(w, B)
    q, k, v, g, b = upload(w, st, (B, T))
    S = dev(s0, "f32")
    o1, s1 = kda.prefill_chunked(q, k, v, g, b, S, state_out=S)
    o2, s2 = kda.prefill_chunked(q, k, v, g, b, dev(s0, "f32"), final_state=False)
    torch.cuda.synchronize()
    assert s1.data_ptr() == S.data_ptr() and s2 is None
    oref, sref = oracle.recurrence(*wide, np.array([0, T]), s0)
    assert_close(host(o1).reshape(T, w.H, w.dv), oref, TOL["bf16"], None, "o (in place)")
    assert_close(host(S), sref, TOL["bf16"], None, "S_T (in place)")
    assert torch.equal(o1, o2), "outputs must not depend on whether the final state is kept"


def test_tiny_workload_exact_shape():
    """The tiny fp32 workload: B=1, H=2, T=64, d=16, chunk 16, zero initial state."""
    w = synth.workload("tiny")
    o, s, oref, sref, cu = _run_prefill(w, 1, w.T, False)
    assert_close(o, oref, 1e-5, cu, "o")
    assert_close(s, sref, 1e-5, None, "S_T")


@pytest.mark.parametrize("dtype,d,N", [
    ("bf16", 128, 6), ("f32", 128, 6), ("f32", 16, 6), ("bf16", 64, 6), ("f32", 32, 6),
    # 130 x 4 = 520 (sequence, head) pairs: one workgroup per pair (the large-batch layout); the
    # cases above split each pair over 16-column workgroups
    ("bf16", 128, 130), ("f32", 64, 130),
])
def test_decode_steps_match_oracle(dtype, d, N):
    print(f"decode dtype={dtype} d={d} N={N}", flush=True)
    w = _w(dtype, H=4, d=d, seed=5, s0_std=0.02)
    w.q_unit = False
    steps = 5
    s0 = synth.gen_state(w, N)
    S = dev(s0, "f32")
    sref = s0.astype(np.float64)
    for t in range(steps):
        st, wide = make_inputs(w, N, offset_tokens=t * N)
        q, k, v, g, b = upload(w, st)
        o = kda.decode_step(q, k, v, g, b, S)  # in place
        torch.cuda.synchronize()
        oref, sref = oracle.decode_step(*wide, sref)
        assert_close(host(o), oref, 1e-5, np.arange(N + 1), f"o step {t}")
    assert_close(host(S), sref, 1e-5, None, "state")


@pytest.mark.parametrize("N", [1, 130])
def test_decode_steps_replayed_from_a_hip_graph_equal_eager_steps(N):
    """Decode steps captured in a HIP graph (the column-split layout at N=1, one workgroup per pair at
    130 x 4 pairs) and replayed three times, with eager calls and synchronisations in between: every
    replay's outputs and final state equal the same steps run eagerly, bit for bit."""
    print(f"decode graph N={N}", flush=True)
    w = _w("bf16", H=4, d=128, seed=9, s0_std=0.02)
    w.q_unit = False
    G = 8
    s0 = dev(synth.gen_state(w, N), "f32")
    steps = []
    for t in range(G):
        st, _ = make_inputs(w, N, offset_tokens=t * N)
        steps.append(upload(w, st))
    Sg = s0.clone()
    outs = [torch.empty(N, w.H, w.dv, device="cuda") for _ in range(G)]

    def run(S, os_):
        for t in range(G):
            kda.decode_step(*steps[t], S, out=os_[t])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(Sg, outs)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(Sg, outs)
    for rep in range(3):
        Se = s0.clone()
        eouts = [torch.empty_like(o) for o in outs]
        run(Se, eouts)  # eager work between the replays
        torch.cuda.synchronize()
        Sg.copy_(s0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Sg, Se), f"state, replay {rep}"
        for t in range(G):
            assert torch.equal(outs[t], eouts[t]), f"output of step {t}, replay {rep}"


def test_decode_out_of_place_equals_in_place():
    w = _w("bf16", H=2, seed=6, s0_std=0.02)
    N = 3
    s0 = synth.gen_state(w, N)
    st, _ = make_inputs(w, N)
    q, k, v, g, b = upload(w, st)
    A = dev(s0, "f32")
    B = dev(s0, "f32")
    Bout = torch.empty_like(B)
    o1 = kda.decode_step(q, k, v, g, b, A)
    o2 = kda.decode_step(q, k, v, g, b, B, state_out=Bout)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(A, Bout)
    assert torch.equal(B, dev(s0, "f32"))  # input untouched


def test_append_varlen_matches_oracle_and_boundaries():
    """Packed segments with empty, one-token, exact-chunk and ragged lengths; distinct carried
    states; canary bytes around the outputs stay untouched."""
    w = _w("bf16", H=3, seed=21, s0_std=0.02)
    lengths = [0, 1, 63, 64, 65, 300, 0, 130]
    cu = synth.cu_seqlens(lengths)
    T, N = int(cu[-1]), len(lengths)
    st, wide = make_inputs(w, T)
    s0 = synth.gen_state(w, N)
    q, k, v, g, b = upload(w, st)
    S0 = dev(s0, "f32")
    canary = 12345.0
    obuf = torch.full((T + 2, w.H, w.dv), canary, device="cuda")
    sbuf = torch.full((N + 2, w.H, w.dk, w.dv), canary, device="cuda")
    o, sT = kda.append_prefill(q, k, v, g, b, torch.from_numpy(cu).cuda(), S0,
                               out=obuf[1:T + 1], state_out=sbuf[1:N + 1])
    torch.cuda.synchronize()
    assert torch.all(obuf[0] == canary) and torch.all(obuf[T + 1] == canary)
    assert torch.all(sbuf[0] == canary) and torch.all(sbuf[N + 1] == canary)
    oref, sref = oracle.recurrence(*wide, cu, s0)
    assert_close(host(o), oref, 2e-3, cu, "o")
    assert_close(host(sT), sref, 2e-3, None, "S_T")
    # empty segments pass their state through bit for bit
    for n in (0, 6):
        assert torch.equal(sT[n], S0[n])


def test_append_isolation_and_determinism():
    """NaN-poisoning one segment leaves every other segment's outputs and states bitwise unchanged;
    two identical calls give identical bits."""
    w = _w("bf16", H=2, seed=31, s0_std=0.02)
    lengths = [70, 129, 5]
    cu = synth.cu_seqlens(lengths)
    T, N = int(cu[-1]), len(lengths)
    st, _ = make_inputs(w, T)
    s0 = synth.gen_state(w, N)
    q, k, v, g, b = upload(w, st)
    cu_d = torch.from_numpy(cu).cuda()
    S0 = dev(s0, "f32")
    o1, s1 = kda.append_prefill(q, k, v, g, b, cu_d, S0)
    o2, s2 = kda.append_prefill(q, k, v, g, b, cu_d, S0)
    v2 = v.clone()
    v2[cu[1]:cu[2]] = float("nan")
    o3, s3 = kda.append_prefill(q, k, v2, g, b, cu_d, S0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert torch.isnan(o3[cu[1]:cu[2]]).any()
    for n in (0, 2):
        assert torch.equal(o3[cu[n]:cu[n + 1]], o1[cu[n]:cu[n + 1]])
        assert torch.equal(s3[n], s1[n])


def test_prefill_equals_append_and_decode_composition():
    """prefill(T1+T2) = append(T2) on the state after prefill(T1), and prefill of T tokens =
    T decode steps, within the bf16-path tolerance."""
    w = _w("bf16", H=2, seed=41)
    T1, T2 = 200, 77
    st, wide = make_inputs(w, T1 + T2)
    q, k, v, g, b = upload(w, st, (1, T1 + T2))
    o, s = kda.prefill_chunked(q, k, v, g, b)
    o1, s1 = kda.prefill_chunked(q[:, :T1].contiguous(), k[:, :T1].contiguous(), v[:, :T1].contiguous(),
                                 g[:, :T1].contiguous(), b[:, :T1].contiguous())
    cu = torch.tensor([0, T2], dtype=torch.int32, device="cuda")
    o2, s2 = kda.append_prefill(q[0, T1:].contiguous(), k[0, T1:].contiguous(), v[0, T1:].contiguous(),
                                g[0, T1:].contiguous(), b[0, T1:].contiguous(), cu, s1)
    torch.cuda.synchronize()
    whole = host(o)[0]
    split = np.concatenate([host(o1)[0], host(o2)])
    assert_close(split, whole, 2e-3, None, "append composition o")
    assert_close(host(s2), host(s), 2e-3, None, "append composition S")
    # decode stepping from zero state over the first 40 tokens
    S = torch.zeros((1, w.H, w.dk, w.dv), device="cuda")
    outs = []
    for t in range(40):
        outs.append(kda.decode_step(q[:, t], k[:, t], v[:, t], g[:, t], b[:, t], S))
    torch.cuda.synchronize()
    dec = np.stack([host(x)[0] for x in outs])
    assert_close(dec, host(o)[0, :40], 2e-3, None, "prefill vs decode")


@pytest.mark.parametrize("gate,head_gate", [
    (synth.Gate("softplus", scale=4.0), False),     # every chunk decays by e^-25 or more over 8 tokens
    (synth.Gate("rate", lo=0.001, hi=8.0), False),  # per-channel rates from weak to very strong
    (synth.Gate("softplus", scale=4.0), True),      # one strong log-decay per token and head
])
def test_strong_decay_matches_oracle(gate, head_gate):
    """Decays beyond the fp16 range of the half-block decay factors (an 8-token decay above e^10 on
    some channel): the matrix-core path sums those chunks' diagonal Gram tiles exactly in fp32,
    and outputs and states match the oracle."""
    print(f"strong decay gate={gate} head_gate={head_gate}", flush=True)
    w = _w("bf16", H=3, seed=51, s0_std=0.02, gate=gate)
    B, T = 2, 333
    st, wide = make_inputs(w, B * T)
    if head_gate:
        st, wide = _head_gate(st, wide)
    assert np.max(-np.asarray(st[3], np.float64)) > 10.0 / 8  # some token needs the exact tiles
    s0 = synth.gen_state(w, B)
    q, k, v, g, b = upload(w, st, (B, T))
    o, sT = kda.prefill_chunked(q, k, v, g, b, dev(s0, "f32"))
    torch.cuda.synchronize()
    cu = np.arange(B + 1) * T
    oref, sref = oracle.recurrence(*wide, cu, s0)
    assert_close(host(o).reshape(B * T, w.H, w.dv), oref, TOL["bf16"], cu, "o")
    assert_close(host(sT), sref, TOL["bf16"], None, "S_T")


def test_strong_and_weak_decay_segments_in_one_call():
    """Packed segments, one of them decaying 40 times faster: the strong chunks take the exact
    diagonal tiles, the weak ones the matrix-core tiles, in the same launch."""
    w = _w("bf16", H=3, seed=53, s0_std=0.02)
    lengths = [200, 130, 64, 77]
    cu = synth.cu_seqlens(lengths)
    T, N = int(cu[-1]), len(lengths)
    print(f"strong and weak segments lengths={lengths}", flush=True)
    st, wide = make_inputs(w, T)
    g = st[3].copy()
    g[cu[1]:cu[2]] *= 40.0
    g[cu[3]:cu[4]] *= 40.0
    st = (st[0], st[1], st[2], g, st[4])
    wide = (wide[0], wide[1], wide[2], g.astype(np.float64), wide[4])
    s0 = synth.gen_state(w, N)
    q, k, v, gd, b = upload(w, st)
    o, sT = kda.append_prefill(q, k, v, gd, b, torch.from_numpy(cu).cuda(), dev(s0, "f32"))
    torch.cuda.synchronize()
    oref, sref = oracle.recurrence(*wide, cu, s0)
    assert_close(host(o), oref, TOL["bf16"], cu, "o")
    assert_close(host(sT), sref, TOL["bf16"], None, "S_T")


# ---------------------------------------------------------------------------------------------
# Gated DeltaNet gate (one log-decay per token and head) and state snapshots
# ---------------------------------------------------------------------------------------------
def _head_gate(st, wide):
    """The same inputs with one gate per head: the first channel's log-decay of each token."""
    q, k, v, g, b = st
    gh = np.ascontiguousarray(g[..., 0])
    return (q, k, v, gh, b), (wide[0], wide[1], wide[2], gh.astype(np.float64), wide[4])


@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 128, 64), ("f32", 32, 32), ("f32", 16, 16), ("bf16", 64, 32)])
def test_head_gate_prefill_and_decode_match_oracle(dtype, d, chunk):
    print(f"head gate dtype={dtype} d={d} chunk={chunk}", flush=True)
    w = _w(dtype, H=3, d=d, chunk=chunk, seed=31, s0_std=0.02)
    B, T = 2, 333
    st, wide = _head_gate(*make_inputs(w, B * T))
    s0 = synth.gen_state(w, B)
    q, k, v, g, b = upload(w, st, (B, T))
    assert g.shape == (B, T, 3)
    o, sT = kda.prefill_chunked(q, k, v, g, b, dev(s0, "f32"), chunk=chunk)
    # one decode step continuing from the prefill's final state, also with a per-head gate
    st2, wide2 = _head_gate(*make_inputs(w, B, offset_tokens=B * T))
    q2, k2, v2, g2, b2 = upload(w, st2)
    S = sT.clone()
    o2 = kda.decode_step(q2, k2, v2, g2, b2, S)
    torch.cuda.synchronize()
    cu = np.arange(B + 1) * T
    oref, sref = oracle.recurrence(*wide, cu, s0)
    assert_close(host(o).reshape(B * T, 3, d), oref, TOL[dtype], cu, "o")
    assert_close(host(sT), sref, TOL[dtype], None, "S_T")
    oref2, sref2 = oracle.recurrence(*wide2, np.arange(B + 1), sref)
    assert_close(host(o2), oref2, TOL[dtype], np.arange(B + 1), "decode o")
    assert_close(host(S), sref2, TOL[dtype], None, "decode S")


@pytest.mark.parametrize("dtype,d,chunk,every", [("bf16", 128, 64, 3), ("f32", 32, 32, 2), ("bf16", 64, 16, 5)])
def test_snapshots_match_oracle(dtype, d, chunk, every):
    """Prefill (B=2, ragged tail) and append (segments shorter than one snapshot interval, empty
    ones and a long one) with state snapshots every `every` chunks."""
    print(f"snapshots dtype={dtype} d={d} chunk={chunk} every={every}", flush=True)
    w = _w(dtype, H=2, d=d, chunk=chunk, seed=37, s0_std=0.02)
    E = every * chunk
    # prefill
    B, T = 2, 1000
    st, wide = make_inputs(w, B * T)
    s0 = synth.gen_state(w, B)
    q, k, v, g, b = upload(w, st, (B, T))
    o, sT, snaps = kda.prefill_chunked(q, k, v, g, b, dev(s0, "f32"), chunk=chunk, snapshot_every=every)
    # append
    lens = [E * 3 + 17, 5, 0, E, E * 2 - 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    Ta = int(cu[-1])
    sta, widea = make_inputs(w, Ta, offset_tokens=B * T)
    s0a = synth.gen_state(w, len(lens))
    qa, ka, va, ga, ba = upload(w, sta)
    oa, sTa, snapsa, snap_cu = kda.append_prefill(qa, ka, va, ga, ba, torch.from_numpy(cu).cuda(), dev(s0a, "f32"),
                                                  chunk=chunk, snapshot_every=every)
    torch.cuda.synchronize()
    assert snaps.shape[:2] == (B, T // E)
    _, _, sref = oracle.recurrence(*wide, np.arange(B + 1) * T, s0, snapshot_every=E)
    assert_close(host(snaps).reshape(-1, 2, d, d), sref, TOL[dtype], None, "prefill snapshots")
    _, sTref, srefa = oracle.recurrence(*widea, cu, s0a, snapshot_every=E)
    assert list(snap_cu.cpu().numpy()) == list(np.concatenate([[0], np.cumsum([n // E for n in lens])]))
    assert srefa.shape[0] == 3 + 0 + 0 + 1 + 1
    assert snapsa.shape[0] == Ta // E >= srefa.shape[0]  # an upper bound: the rows are counted on the device
    assert_close(host(snapsa[:srefa.shape[0]]), srefa, TOL[dtype], None, "append snapshots")
    assert_close(host(sTa), sTref, TOL[dtype], None, "append S_T")


# ---------------------------------------------------------------------------------------------
# Fused input prologue: raw q, k (normalised in the kernels), beta logits, raw gate inputs
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,d,chunk,gate_head,scale", [
    ("bf16", 128, 64, False, 0.1), ("bf16", 128, 64, True, 0.1), ("f32", 32, 32, False, 0.1),
    ("f32", 16, 16, True, 0.1),
    ("bf16", 128, 64, False, 4.0),  # strong decays: the exact diagonal tiles, from raw gate inputs
])
def test_fused_prologue_matches_oracle(dtype, d, chunk, gate_head, scale):
    print(f"prologue dtype={dtype} d={d} chunk={chunk} gate_head={gate_head} scale={scale}", flush=True)
    w = _w(dtype, H=3, d=d, chunk=chunk, seed=43, s0_std=0.02)
    B, T = 2, 333
    q, k, v, a, b = synth.gen_raw_tokens(w, B * T + B, gate_head=gate_head)
    s0 = synth.gen_state(w, B)
    wide = [synth.to_f64(x, dtype) for x in (q, k, v)] + [a.astype(np.float64), synth.to_f64(b, dtype)]
    qn, kn, beta, g = oracle.prologue(wide[0], wide[1], wide[4], wide[3], scale)
    tq, tk, tv, tb = (dev(x, dtype) for x in (q, k, v, b))
    ta = dev(a, "f32")
    n = B * T
    bt = lambda t: t[:n].reshape(B, T, *t.shape[1:])  # noqa: E731
    o, sT = kda.prefill_chunked(bt(tq), bt(tk), bt(tv), bt(ta), bt(tb), dev(s0, "f32"), chunk=chunk,
                                prologue_gate_scale=scale)
    S = sT.clone()
    o2 = kda.decode_step(tq[n:], tk[n:], tv[n:], ta[n:], tb[n:], S, prologue_gate_scale=scale)
    torch.cuda.synchronize()
    cu = np.arange(B + 1) * T
    oref, sref = oracle.recurrence(qn[:n], kn[:n], wide[2][:n], g[:n], beta[:n], cu, s0)
    assert_close(host(o).reshape(n, 3, d), oref, TOL[dtype], cu, "o")
    assert_close(host(sT), sref, TOL[dtype], None, "S_T")
    oref2, sref2 = oracle.recurrence(qn[n:], kn[n:], wide[2][n:], g[n:], beta[n:], np.arange(B + 1), sref)
    assert_close(host(o2), oref2, TOL[dtype], np.arange(B + 1), "decode o")
    assert_close(host(S), sref2, TOL[dtype], None, "decode S")
