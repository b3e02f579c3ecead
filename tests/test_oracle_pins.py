"""Pins of the fp64 oracle to what the pages and mathematics fix (CPU only).

Pages: "Kimi K3, explained" (vibeengines.com/paper/kimi-k3).  Each test names the section it
follows.  Each pin is chosen so that a plausible mistake in the oracle fails it:
  dropped erase / wrong sign of the correction      -> overwrite example, Widrow-Hoff form
  decay applied after the write, or read before it  -> overwrite under any decay, first read
  decay along the value axis, alpha used as log     -> decay-only closed form
  beta missing on the write or on the erase         -> two-write closed form
  chunk or sequence boundary mistakes               -> chunked algebra, append composition
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")
pytestmark = pytest.mark.timeout(300)


def _one_head(qs, ks, vs, gs, bs, s0=None):
    """Run the oracle on a single sequence and head; per-token lists -> (o [T,dv], S [dk,dv])."""
    q = np.asarray(qs, np.float64)[:, None, :]
    k = np.asarray(ks, np.float64)[:, None, :]
    v = np.asarray(vs, np.float64)[:, None, :]
    g = np.asarray(gs, np.float64)[:, None, :]
    b = np.asarray(bs, np.float64)[:, None]
    S0 = None if s0 is None else np.asarray(s0, np.float64)[None, None]
    o, sT = oracle.recurrence(q, k, v, g, b, None, S0, threads=1)
    return o[:, 0, :], sT[0, 0]


def _rand_unit(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ---------------------------------------------------------------------------------------------
# (a) the page's overwrite example ("The delta: overwrite, don't accumulate"; "Solve it
#     yourself"; first "Check yourself" answer)
# ---------------------------------------------------------------------------------------------
def test_overwrite_example_golden():
    ex = json.load(open(os.path.join(GOLD, "p3_overwrite_example.json")))
    D = ex["D"]
    k1 = np.eye(D)[ex["key_index"]]
    a, b = np.array(ex["a"]), np.array(ex["b"])
    zero = np.zeros(D)
    # two writes under the same unit key, beta = 1, no decay (g = 0); read with q = k1
    o, S = _one_head([k1, k1], [k1, k1], [a, b], [zero, zero], [1.0, 1.0])
    np.testing.assert_array_equal(o[1], ex["delta_read_after_two_writes"])
    np.testing.assert_array_equal(S.T @ k1, ex["delta_read_after_two_writes"])
    np.testing.assert_array_equal(o[0], a)  # write a key, read it back
    # plain linear attention accumulates: a + b
    ol, Sl = oracle.linear_attention(np.stack([k1, k1]), np.stack([k1, k1]), np.stack([a, b]))
    np.testing.assert_array_equal(ol[1], ex["linear_read_after_two_writes"])
    assert not np.array_equal(o[1], ol[1])


def test_runnable_assertions_distinct_keys_and_fixed_state():
    """The runnable's assertions: distinct keys do not interfere; the state is d x d whatever
    the context length."""
    D = 4
    k1, k2 = np.eye(D)[1], np.eye(D)[2]
    a, b = np.array([9.0, 8.0, 7.0, 6.0]), np.array([1.0, 2.0, 3.0, 4.0])
    z = np.zeros(D)
    o, S = _one_head([k1, k2], [k1, k2], [a, b], [z, z], [1.0, 1.0])
    np.testing.assert_array_equal(S.T @ k1, a)
    np.testing.assert_array_equal(S.T @ k2, b)
    for T in (1, 10, 300):
        rng = np.random.default_rng(T)
        q, k = _rand_unit(rng, T, D), _rand_unit(rng, T, D)
        _, S = _one_head(q, k, rng.standard_normal((T, D)), -0.1 * rng.random((T, D)), rng.random(T))
        assert S.shape == (D, D)


def test_state_size_golden():
    ex = json.load(open(os.path.join(GOLD, "decay_and_state_size.json")))["state_size"]
    dk, dv = ex["d_k"], ex["d_v"]
    rng = np.random.default_rng(0)
    T = 3
    q, k = _rand_unit(rng, T, dk), _rand_unit(rng, T, dk)
    _, S = _one_head(q, k, rng.standard_normal((T, dv)), np.zeros((T, dk)), np.ones(T))
    assert S.size == ex["state_numbers_per_head"]
    assert round(ex["softmax_numbers_per_head_after_1M_tokens"] / S.size, -2) == ex["ratio_about"]


# ---------------------------------------------------------------------------------------------
# (a') "The math", special cases: beta = 1 and a unit key -> reading k right after the write
#      returns exactly v, for any decay and any prior state.
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_overwrite_under_any_decay(seed):
    rng = np.random.default_rng(seed)
    dk, dv, T = 12, 7, 20
    k = _rand_unit(rng, T, dk)
    v = rng.standard_normal((T, dv))
    g = np.log(rng.uniform(0.05, 1.0, (T, dk)))
    S0 = rng.standard_normal((dk, dv))
    o, _ = _one_head(k, k, v, g, np.ones(T), S0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)
    # the pin has teeth: the same data with beta = 0.7 does not overwrite
    o2, _ = _one_head(k, k, v, g, 0.7 * np.ones(T), S0)
    assert np.abs(o2 - v).max() > 1e-3


def test_two_writes_closed_form():
    """Unit key, no decay, strengths b1 then b2: the first write leaves b1*a under k; the second
    erases a b2 share of it and adds b2*b, so the read is (1-b2)*b1*a + b2*b
    ("How Kimi Delta Attention works, step by step": erase, then write)."""
    rng = np.random.default_rng(7)
    dk, dv = 9, 5
    k = _rand_unit(rng, 1, dk)[0]
    a, b = rng.standard_normal(dv), rng.standard_normal(dv)
    for b1, b2 in [(0.3, 0.6), (1.0, 0.25), (0.5, 0.0), (0.9, 1.0)]:
        o, S = _one_head([k, k], [k, k], [a, b], np.zeros((2, dk)), [b1, b2])
        np.testing.assert_allclose(o[0], b1 * a, rtol=0, atol=1e-13)
        np.testing.assert_allclose(o[1], (1 - b2) * b1 * a + b2 * b, rtol=0, atol=1e-13)
    # a read with a query other than the key: first write from zero gives o = beta (k.q) v
    q = rng.standard_normal(dk)
    o, _ = _one_head([q], [k], [a], [np.zeros(dk)], [0.4])
    np.testing.assert_allclose(o[0], 0.4 * (k @ q) * a, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------------------------
# (b) beta = 0 and alpha = 1: nothing is written and nothing fades.
# ---------------------------------------------------------------------------------------------
def test_no_write_identity():
    rng = np.random.default_rng(3)
    dk, dv, T = 16, 16, 40
    S0 = rng.standard_normal((dk, dv))
    q = rng.standard_normal((T, dk))
    o, S = _one_head(q, _rand_unit(rng, T, dk), rng.standard_normal((T, dv)), np.zeros((T, dk)), np.zeros(T), S0)
    np.testing.assert_array_equal(S, S0)
    np.testing.assert_allclose(o, q @ S0, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------------------------
# (b') beta = 0: the state only fades, S_T = Diag(exp(sum_t g_t)) S0 — per key channel.
#      Golden: alpha = 0.5 for 10 tokens leaves 0.5^10 ~ 0.001; alpha ~ 1 leaves ~ all
#      (third "Check yourself" question).
# ---------------------------------------------------------------------------------------------
def test_decay_only_closed_form():
    ex = json.load(open(os.path.join(GOLD, "decay_and_state_size.json")))["decay"]
    rng = np.random.default_rng(4)
    dk, dv, T = 8, 8, ex["tokens"]
    g = np.tile(np.log(rng.uniform(0.2, 1.0, dk)), (T, 1))
    g[:, 0] = np.log(ex["alpha"])
    g[:, 1] = 0.0
    S0 = rng.standard_normal((dk, dv))
    _, S = _one_head(rng.standard_normal((T, dk)), _rand_unit(rng, T, dk), rng.standard_normal((T, dv)), g,
                     np.zeros(T), S0)
    np.testing.assert_allclose(S, np.exp(g.sum(0))[:, None] * S0, rtol=1e-13, atol=0)
    frac = S[0] / S0[0]
    np.testing.assert_allclose(frac, ex["remaining_exact"], rtol=1e-13)
    assert abs(frac[0] - ex["page_says_about"]) < 1e-4
    np.testing.assert_allclose(S[1] / S0[1], ex["alpha_near_one_remaining"], rtol=1e-15)


# ---------------------------------------------------------------------------------------------
# (c) non-expansive: |k| = 1, beta in [0,1], alpha in (0,1] -> two initial states do not move
#     apart (||I - beta k k^T|| = 1, ||Diag alpha|| <= 1), in Frobenius norm and per column.
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_non_expansive(seed):
    rng = np.random.default_rng(seed)
    dk, dv, T = 10, 6, 60
    q, k = rng.standard_normal((T, dk)), _rand_unit(rng, T, dk)
    v = rng.standard_normal((T, dv))
    g = np.log(rng.uniform(0.3, 1.0, (T, dk)))
    g[rng.random((T, dk)) < 0.3] = 0.0  # some channels do not decay
    b = rng.uniform(0, 1, T)
    b[::7] = 1.0
    S0, S1 = rng.standard_normal((dk, dv)), rng.standard_normal((dk, dv))
    _, A = _one_head(q, k, v, g, b, S0)
    _, B = _one_head(q, k, v, g, b, S1)
    assert np.linalg.norm(A - B) <= np.linalg.norm(S0 - S1) + 1e-12
    assert np.all(np.linalg.norm(A - B, axis=0) <= np.linalg.norm(S0 - S1, axis=0) + 1e-12)


def test_non_expansive_has_teeth():
    """Outside the stated range (beta = 2.5 -> eigenvalue -1.5 along k) the map expands."""
    rng = np.random.default_rng(11)
    dk, dv, T = 6, 3, 30
    k = _rand_unit(rng, T, dk)
    S0, S1 = rng.standard_normal((dk, dv)), rng.standard_normal((dk, dv))
    args = (rng.standard_normal((T, dk)), k, rng.standard_normal((T, dv)), np.zeros((T, dk)), 2.5 * np.ones(T))
    _, A = _one_head(*args, S0)
    _, B = _one_head(*args, S1)
    assert np.linalg.norm(A - B) > np.linalg.norm(S0 - S1)


# ---------------------------------------------------------------------------------------------
# (d) the chunked algebra ("Training in chunks") reaches the recurrence's result.
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("chunk", [1, 5, 16, 64])
def test_chunked_matches_recurrence(chunk):
    rng = np.random.default_rng(chunk)
    H, dk, dv = 2, 16, 12
    lengths = [37, 0, 64, 1, 20]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T = int(cu[-1])
    q, k = _rand_unit(rng, T * H, dk).reshape(T, H, dk), _rand_unit(rng, T * H, dk).reshape(T, H, dk)
    v = rng.standard_normal((T, H, dv))
    g = -0.3 * np.log1p(np.exp(rng.standard_normal((T, H, dk))))
    b = 1 / (1 + np.exp(-rng.standard_normal((T, H))))
    s0 = 0.5 * rng.standard_normal((len(lengths), H, dk, dv))
    o1, s1 = oracle.recurrence(q, k, v, g, b, cu, s0)
    o2, s2 = oracle.chunked(q, k, v, g, b, cu, s0, chunk=chunk)
    assert np.abs(o1 - o2).max() <= 1e-12 * max(1.0, np.abs(o1).max())
    assert np.abs(s1 - s2).max() <= 1e-12 * max(1.0, np.abs(s1).max())


# ---------------------------------------------------------------------------------------------
# Further properties fixed by the definition
# ---------------------------------------------------------------------------------------------
def test_orthonormal_keys_no_interference():
    """alpha = 1, beta = 1, orthonormal keys: each read returns its own value (runnable assertion 3)."""
    rng = np.random.default_rng(5)
    d = 16
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Qm.T  # rows orthonormal
    vals = rng.standard_normal((d, d))
    _, S = _one_head(keys, keys, vals, np.zeros((d, d)), np.ones(d))
    np.testing.assert_allclose(keys @ S, vals, atol=1e-12)


def test_linearity_in_values_and_state():
    rng = np.random.default_rng(6)
    T, H, dk, dv = 30, 2, 8, 5
    q, k = rng.standard_normal((T, H, dk)), _rand_unit(rng, T * H, dk).reshape(T, H, dk)
    g = np.log(rng.uniform(0.5, 1, (T, H, dk)))
    b = rng.random((T, H))
    V1, V2 = rng.standard_normal((T, H, dv)), rng.standard_normal((T, H, dv))
    S1, S2 = rng.standard_normal((1, H, dk, dv)), rng.standard_normal((1, H, dk, dv))
    c1, c2 = 0.7, -1.3
    o, s = oracle.recurrence(q, k, c1 * V1 + c2 * V2, g, b, None, c1 * S1 + c2 * S2)
    oa, sa = oracle.recurrence(q, k, V1, g, b, None, S1)
    ob, sb = oracle.recurrence(q, k, V2, g, b, None, S2)
    np.testing.assert_allclose(o, c1 * oa + c2 * ob, atol=1e-12)
    np.testing.assert_allclose(s, c1 * sa + c2 * sb, atol=1e-12)


def test_independence_of_columns_heads_sequences():
    rng = np.random.default_rng(8)
    T, H, dk, dv = 25, 3, 6, 7
    q, k = rng.standard_normal((T, H, dk)), _rand_unit(rng, T * H, dk).reshape(T, H, dk)
    v, g, b = rng.standard_normal((T, H, dv)), np.log(rng.uniform(0.5, 1, (T, H, dk))), rng.random((T, H))
    o, s = oracle.recurrence(q, k, v, g, b)
    perm = rng.permutation(dv)
    op, sp = oracle.recurrence(q, k, v[:, :, perm], g, b)
    np.testing.assert_array_equal(op, o[:, :, perm])
    np.testing.assert_array_equal(sp, s[..., perm])
    v2 = v.copy()
    v2[:, 1] = 1e3 * rng.standard_normal((T, dv))
    o2, s2 = oracle.recurrence(q, k, v2, g, b)
    np.testing.assert_array_equal(o2[:, [0, 2]], o[:, [0, 2]])
    cu = [0, 10, 25]
    o3, s3 = oracle.recurrence(q, k, v, g, b, cu)
    o4, s4 = oracle.recurrence(q[10:], k[10:], v[10:], g[10:], b[10:])
    np.testing.assert_array_equal(o3[10:], o4)
    np.testing.assert_array_equal(s3[1], s4[0])


def test_append_and_decode_composition():
    """Prefill of T1+T2 tokens = append of T2 tokens on the state after T1; one decode step is a
    one-token prefill (the append-prefill workload of the first page; decode per "The decode wall")."""
    rng = np.random.default_rng(9)
    T, H, dk, dv = 48, 2, 8, 8
    q, k = rng.standard_normal((T, H, dk)), _rand_unit(rng, T * H, dk).reshape(T, H, dk)
    v, g, b = rng.standard_normal((T, H, dv)), np.log(rng.uniform(0.5, 1, (T, H, dk))), rng.random((T, H))
    o, s = oracle.recurrence(q, k, v, g, b)
    o1, s1 = oracle.recurrence(q[:30], k[:30], v[:30], g[:30], b[:30])
    o2, s2 = oracle.recurrence(q[30:], k[30:], v[30:], g[30:], b[30:], None, s1)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(s2, s, rtol=0, atol=1e-13)
    od, sd = oracle.decode_step(q[30][None], k[30][None], v[30][None], g[30][None], b[30][None], s1)
    np.testing.assert_allclose(od[0], o[30], atol=1e-13)


def test_matches_both_orientations_of_the_equation():
    """Cross-check (not a pin: it restates the equation) — the page's d_v x d_k form
    S_t = S_{t-1} Diag(alpha)(I - beta k k^T) + beta v k^T, o = S q, transposed, equals the oracle."""
    rng = np.random.default_rng(10)
    T, dk, dv = 12, 5, 4
    q, k = rng.standard_normal((T, dk)), _rand_unit(rng, T, dk)
    v, g, b = rng.standard_normal((T, dv)), np.log(rng.uniform(0.3, 1, (T, dk))), rng.random(T)
    o, S = _one_head(q, k, v, g, b)
    P = np.zeros((dv, dk))
    for t in range(T):
        P = P @ np.diag(np.exp(g[t])) @ (np.eye(dk) - b[t] * np.outer(k[t], k[t])) + b[t] * np.outer(v[t], k[t])
        np.testing.assert_allclose(P @ q[t], o[t], atol=1e-12)
    np.testing.assert_allclose(P.T, S, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# Gated DeltaNet: one forget gate per head and token ("Kimi K3, explained", the comparison of
# KDA with Gated DeltaNet: a scalar decay instead of one per key channel)
# ---------------------------------------------------------------------------------------------
def test_head_gate_decay_only_closed_form():
    """beta = 0 with a per-head gate: the whole state shrinks by exp(sum of g) (every channel
    alike, unlike the per-channel case above)."""
    rng = np.random.default_rng(21)
    T, H, dk, dv = 12, 3, 8, 6
    g = np.log(rng.uniform(0.3, 1.0, (T, H)))
    S0 = rng.standard_normal((1, H, dk, dv))
    _, S = oracle.recurrence(rng.standard_normal((T, H, dk)), _rand_unit(rng, T * H, dk).reshape(T, H, dk),
                             rng.standard_normal((T, H, dv)), g, np.zeros((T, H)), None, S0, threads=1)
    np.testing.assert_allclose(S[0], np.exp(g.sum(0))[:, None, None] * S0[0], rtol=1e-13, atol=0)


def test_head_gate_overwrite_under_any_decay():
    """beta = 1, unit key: whatever the scalar decay and the prior state, reading the key right
    after the write returns the written value ("The math", the overwrite special case)."""
    rng = np.random.default_rng(22)
    T, H, dk, dv = 9, 2, 8, 5
    k = _rand_unit(rng, T * H, dk).reshape(T, H, dk)
    v = rng.standard_normal((T, H, dv))
    o, _ = oracle.recurrence(k, k, v, np.log(rng.uniform(0.05, 1.0, (T, H))), np.ones((T, H)), None,
                             rng.standard_normal((1, H, dk, dv)), threads=1)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# State snapshots ("Kimi K3 changed the memory math for agentic AI": checkpoints of the
# fixed-size state along a long context): snapshot m of a sequence is the state after its
# first (m + 1) * E tokens, i.e. the final state of a run over just those tokens.
# ---------------------------------------------------------------------------------------------
def test_snapshots_are_final_states_of_prefixes():
    rng = np.random.default_rng(23)
    H, dk, dv, E = 2, 8, 6, 7
    lens = [30, 5, 0, 21, 14]  # with a sequence shorter than E and an empty one
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q = rng.standard_normal((T, H, dk))
    k = _rand_unit(rng, T * H, dk).reshape(T, H, dk)
    v = rng.standard_normal((T, H, dv))
    g = np.log(rng.uniform(0.5, 1.0, (T, H, dk)))
    b = rng.uniform(0, 1, (T, H))
    s0 = rng.standard_normal((len(lens), H, dk, dv))
    _, sT, snaps = oracle.recurrence(q, k, v, g, b, cu, s0, threads=2, snapshot_every=E)
    assert snaps.shape[0] == sum(n // E for n in lens)
    row = 0
    for n, L in enumerate(lens):
        for m in range(L // E):
            sl = slice(cu[n], cu[n] + (m + 1) * E)
            _, ref = oracle.recurrence(q[sl], k[sl], v[sl], g[sl], b[sl], None, s0[n:n + 1], threads=1)
            np.testing.assert_allclose(snaps[row], ref[0], rtol=0, atol=0)
            row += 1
    # a snapshot exactly at the end of a sequence equals its final state (sequences 3 and 4:
    # rows 4..6 and 7..8)
    np.testing.assert_allclose(snaps[6], sT[3], rtol=0, atol=0)
    np.testing.assert_allclose(snaps[8], sT[4], rtol=0, atol=0)


# ---------------------------------------------------------------------------------------------
# Fused input prologue ("Kimi K3, explained", "How Kimi Delta Attention works, step by step":
# normalised queries and keys, beta and alpha in (0, 1))
# ---------------------------------------------------------------------------------------------
def test_prologue_closed_forms():
    rng = np.random.default_rng(24)
    q, k = rng.standard_normal((2, 5, 3, 16)) * 7.0
    k[0, 0] = 0.0  # a zero key stays zero
    qn, kn, beta, g = oracle.prologue(q, k, np.array([0.0, 40.0, -40.0, 3.0]), np.array([0.0, 50.0, -50.0, 1.0]),
                                      0.1)
    np.testing.assert_allclose(np.linalg.norm(qn, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(np.linalg.norm(kn[1:], axis=-1), 1.0, rtol=1e-14)
    assert np.all(kn[0, 0] == 0.0)
    np.testing.assert_allclose(kn * np.linalg.norm(k, axis=-1, keepdims=True), k, rtol=1e-14, atol=0)
    # sigmoid: 1/2 at 0, saturating at +-40; 3 -> e^3 / (1 + e^3)
    np.testing.assert_allclose(beta, [0.5, 1.0, np.exp(-40.0), np.exp(3.0) / (1 + np.exp(3.0))], rtol=1e-14)
    # softplus: ln 2 at 0, x for large x, e^x for very negative x, log(1 + e) at 1
    np.testing.assert_allclose(g, [-0.1 * np.log(2.0), -5.0, -0.1 * np.exp(-50.0), -0.1 * np.log1p(np.e)],
                               rtol=1e-14)
