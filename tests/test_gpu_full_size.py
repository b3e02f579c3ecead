"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

The oracle recomputes sampled (sequence, head) slices token by token in fp64 (value columns
split across host threads); the GPU runs the whole workload.  Tolerance per slice:
max|gpu - oracle| / max|oracle| <= 2e-3 (bfloat16 storage, fp32 state).

Workloads (seeded, see synth.workload):
  prefill  B=1, H=32, T=8192, d=128, chunk 64, zero initial state   (every head checked)
  metric   the same at T=65,536 (the headline prefill)              (every head checked)
  decode   256 sequences x 32 heads, 1000 in-place steps            (every pair at the first step;
                                                                     8 pairs at every step)
  varlen   8 carried states, segments of 1K..32K tokens, packed     (every head, every segment)
  long     B=1, H=32, T=2^20, per-channel rates, then 4096 decode steps (4 heads, every token);
           its backward (windowed) on one head's last 1,024 tokens
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_75_amd as kda
import oracle
import synth
from _gpu import dev, host
from _util import assert_close

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
TOL = 2e-3


def _wide(x, dt):
    return synth.to_f64(x, dt)


def _heads(st, heads, dt):
    q, k, v, g, b = st
    return (_wide(q[:, heads], dt), _wide(k[:, heads], dt), _wide(v[:, heads], dt),
            g[:, heads].astype(np.float64), _wide(b[:, heads], dt))


def _prefill_full(w, T, heads, threads=None):
    print(f"[{w.name}] generate T={T} H={w.H}", flush=True)
    st = synth.gen_tokens(w, T)
    q, k, v, g, b = st
    tq, tk, tv, tb = (dev(x, "bf16").reshape(1, T, *x.shape[1:]) for x in (q, k, v, b))
    tg = dev(g, "f32").reshape(1, T, w.H, w.dk)
    print(f"[{w.name}] gpu prefill", flush=True)
    o, sT = kda.prefill_chunked(tq, tk, tv, tg, tb)
    torch.cuda.synchronize()
    del tq, tk, tv, tb, tg
    print(f"[{w.name}] oracle on heads {heads}", flush=True)
    vcols = 8 if len(heads) < 4 else 32
    oref, sref = oracle.recurrence(*_heads(st, heads, "bf16"), vcols=vcols)
    og = host(o[0][:, heads])
    sg = host(sT[:, heads])
    return st, o, sT, og, sg, oref, sref


def test_prefill_workload_all_heads():
    w = synth.workload("prefill")
    heads = list(range(w.H))
    _, _, _, og, sg, oref, sref = _prefill_full(w, w.T, heads)
    assert_close(og, oref, TOL, None, "o")
    assert_close(sg, sref, TOL, None, "S_T")


def test_metric_prefill_sampled_heads():
    w = synth.workload("metric")
    heads = list(range(w.H))
    _, o, sT, og, sg, oref, sref = _prefill_full(w, w.T, heads)
    assert_close(og, oref, TOL, None, "o")
    assert_close(sg, sref, TOL, None, "S_T")
    assert torch.isfinite(o).all() and torch.isfinite(sT).all()


def test_decode_workload_1000_steps():
    w = synth.workload("decode")
    N, H, steps = w.decode_N, w.H, w.decode_steps
    print(f"[decode] generate {steps} steps x {N} x {H}", flush=True)
    q, k, v, g, b = synth.gen_tokens(w, steps * N)
    s0 = synth.gen_state(w, N)
    tq, tk, tv, tb = (dev(x, "bf16").reshape(steps, N, *x.shape[1:]) for x in (q, k, v, b))
    tg = dev(g, "f32").reshape(steps, N, H, w.dk)
    S = dev(s0, "f32")
    pairs = [(0, 0), (3, 31), (77, 7), (128, 16), (200, 1), (255, 30), (31, 13), (150, 25)]
    pn = torch.tensor([p[0] for p in pairs], device="cuda")
    ph = torch.tensor([p[1] for p in pairs], device="cuda")
    outs = torch.empty((steps, len(pairs), w.dv), device="cuda")
    out = torch.empty((N, H, w.dv), device="cuda")
    # the first step on every (sequence, head) pair, out of place, against the oracle's step
    S1 = torch.empty_like(S)
    kda.decode_step(tq[0], tk[0], tv[0], tg[0], tb[0], S, out=out, state_out=S1)
    torch.cuda.synchronize()
    wide0 = (_wide(q[:N], "bf16"), _wide(k[:N], "bf16"), _wide(v[:N], "bf16"), g[:N].astype(np.float64),
             _wide(b[:N], "bf16"))
    print("[decode] oracle step 0 on all pairs", flush=True)
    o0, s1 = oracle.decode_step(*wide0, s0.astype(np.float64))
    assert_close(host(out), o0, TOL, np.arange(N + 1), "o step 0, all pairs")
    assert_close(host(S1), s1, TOL, None, "S step 0, all pairs")
    del S1, s1
    print("[decode] gpu steps", flush=True)
    for t in range(steps):
        kda.decode_step(tq[t], tk[t], tv[t], tg[t], tb[t], S, out=out)
        outs[t] = out[pn, ph]
    torch.cuda.synchronize()
    og, Sg = host(outs), host(S)
    assert torch.isfinite(S).all()
    print("[decode] oracle", flush=True)
    for i, (n, h) in enumerate(pairs):
        def sl(x):
            return x.reshape(steps, N, H, -1)[:, n, h]
        wide = (_wide(sl(q), "bf16")[:, None], _wide(sl(k), "bf16")[:, None], _wide(sl(v), "bf16")[:, None],
                sl(g).astype(np.float64)[:, None], _wide(b.reshape(steps, N, H)[:, n, h], "bf16")[:, None])
        oref, sref = oracle.recurrence(*wide, None, s0[n, h][None, None].astype(np.float64), threads=1)
        assert_close(og[:, i][:, None, :], oref, TOL, None, f"o pair {(n, h)}")
        assert_close(Sg[n, h][None, None], sref, TOL, None, f"S pair {(n, h)}")


def test_varlen_append_workload():
    w = synth.workload("varlen")
    cu = synth.cu_seqlens(w.lengths)
    T, N = int(cu[-1]), len(w.lengths)
    print(f"[varlen] generate T_total={T} lengths={w.lengths}", flush=True)
    st = synth.gen_tokens(w, T)
    q, k, v, g, b = st
    s0 = synth.gen_state(w, N)
    o, sT = kda.append_prefill(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(g, "f32"), dev(b, "bf16"),
                               torch.from_numpy(cu).cuda(), dev(s0, "f32"))
    torch.cuda.synchronize()
    heads = list(range(w.H))
    print(f"[varlen] oracle on heads {heads}", flush=True)
    oref, sref = oracle.recurrence(*_heads(st, heads, "bf16"), cu, s0[:, heads], vcols=32)
    assert_close(host(o[:, heads]), oref, TOL, cu, "o")
    assert_close(host(sT[:, heads]), sref, TOL, None, "S_T")
    assert torch.isfinite(o).all() and torch.isfinite(sT).all()


@pytest.mark.timeout(900)
def test_long_context_prefill_then_decode():
    w = synth.workload("long")
    T, H, steps = w.T, w.H, w.decode_steps
    heads = [0, 11, 20, 31]
    st, o, sT, og, sg, oref, sref = _prefill_full(w, T, heads)
    assert_close(og, oref, TOL, None, "o (1M prefill)")
    assert_close(sg, sref, TOL, None, "S_T (1M prefill)")
    assert torch.isfinite(o).all() and torch.isfinite(sT).all()
    del o, st, og, oref
    # decode continues the same token stream from the prefill's final state
    print(f"[long] {steps} decode steps", flush=True)
    dq, dk_, dv_, dg, db = synth.gen_tokens(w, steps, offset_tokens=T)
    tq, tk, tv, tb = (dev(x, "bf16") for x in (dq, dk_, dv_, db))
    tg = dev(dg, "f32")
    S = sT.clone()
    outs = torch.empty((steps, H, w.dv), device="cuda")
    for t in range(steps):
        outs[t] = kda.decode_step(tq[t:t + 1], tk[t:t + 1], tv[t:t + 1], tg[t:t + 1], tb[t:t + 1], S)[0]
    torch.cuda.synchronize()
    oref2, sref2 = oracle.recurrence(*_heads((dq, dk_, dv_, dg, db), heads, "bf16"), None, sref, vcols=32)
    assert_close(host(outs[:, heads]), oref2, TOL, None, "o (decode tail)")
    assert_close(host(S[:, heads]), sref2, TOL, None, "S (decode tail)")


def _backward_full(w, T, heads, with_state):
    """The chunked backward over all heads of a T-token sequence (the launch bench.py times: B=1, bf16
    inputs, chunk 64); the oracle's derivative on the sampled heads."""
    print(f"[{w.name}] backward: generate T={T} H={w.H}", flush=True)
    q, k, v, g, b = synth.gen_tokens(w, T)
    s0 = synth.gen_state(w, 1) if with_state else None
    d_out, d_sT = synth.gen_cotangents(w, T, 1)
    cu = np.array([0, T], np.int32)
    print(f"[{w.name}] gpu backward", flush=True)
    grads = kda.chunked_backward(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(g, "f32"), dev(b, "bf16"),
                                 torch.from_numpy(cu).cuda(), dev(s0, "f32") if s0 is not None else None,
                                 d_out=dev(d_out, "f32"), d_state_out=dev(d_sT, "f32"), chunk=w.chunk)
    torch.cuda.synchronize()
    for x in grads:
        assert torch.isfinite(x).all()
    got = [host(x[:, heads]) for x in grads]
    print(f"[{w.name}] oracle backward on heads {heads}", flush=True)
    ref = oracle.backward(*_heads((q, k, v, g, b), heads, "bf16"), cu,
                          s0[:, heads] if s0 is not None else None, d_o=d_out[:, heads], d_sT=d_sT[:, heads])
    for name, x, y in zip(("dq", "dk", "dv", "dg", "dbeta"), got[:5], ref[:5]):
        if x.ndim == 2:
            x, y = x[:, :, None], y[:, :, None]
        assert_close(x, y, TOL, cu, name)
    assert_close(got[5], ref[5], TOL, None, "dS0")


def test_backward_prefill_workload_all_heads():
    """Gradients at the prefill workload's size (T=8192, H=32), every head, with a carried state."""
    w = synth.workload("prefill")
    w.s0_std = 0.02
    _backward_full(w, w.T, list(range(w.H)), True)


@pytest.mark.timeout(600)
def test_backward_metric_sampled_heads():
    """Gradients at the headline prefill's size (T=65,536, H=32), two heads checked."""
    w = synth.workload("metric")
    _backward_full(w, w.T, [3, 28], False)


@pytest.mark.timeout(900)
def test_backward_long_context_last_tokens():
    """The chunked backward of the 2^20-token workload (all 32 heads; its one-pass workspace would
    be about 274 GiB, so it runs in windows under the 20 GiB cap), checked on one head's last 1,024
    tokens: the oracle's derivative over those tokens, started from the oracle's own state after
    the first 2^20 - 1,024 tokens, with the same dL/do and dL/dS_T."""
    from gated_delta_rule_75_amd import _lib

    w = synth.workload("long")
    T, H, d, n, h = w.T, w.H, w.dk, 1024, 11
    ws = kda.workspace_size(_lib.KDA_OP_BACKWARD, 1, T, H, d, d, torch.bfloat16, 64)
    assert ws <= 24 << 30
    print(f"[long] backward: generate T={T} H={H} (workspace {ws / 2**30:.1f} GiB)", flush=True)
    q, k, v, g, b = synth.gen_tokens(w, T)
    d_out, d_sT = synth.gen_cotangents(w, T, 1)
    cu = np.array([0, T], np.int32)
    print("[long] gpu backward", flush=True)
    grads = kda.chunked_backward(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(g, "f32"), dev(b, "bf16"),
                                 torch.from_numpy(cu).cuda(), None, d_out=dev(d_out, "f32"),
                                 d_state_out=dev(d_sT, "f32"), chunk=64, state_grad=False)
    torch.cuda.synchronize()
    got = [host(x[T - n:, h:h + 1]) for x in grads[:5]]
    for x in grads[:5]:
        assert torch.isfinite(x).all()
    del grads
    torch.cuda.empty_cache()
    print(f"[long] oracle: forward over {T - n} tokens, derivative over the last {n} (head {h})", flush=True)
    wide = _heads((q, k, v, g, b), [h], "bf16")
    del q, k, v, g, b
    _, s_mid = oracle.recurrence(*(x[:T - n] for x in wide), vcols=8)
    ref = oracle.backward(*(x[T - n:] for x in wide), None, s_mid, d_o=d_out[T - n:, h:h + 1],
                          d_sT=d_sT[:, h:h + 1])
    for name, x, y in zip(("dq", "dk", "dv", "dg", "dbeta"), got, ref[:5]):
        if x.ndim == 2:
            x, y = x[:, :, None], y[:, :, None]
        assert_close(x, y, TOL, None, name)
