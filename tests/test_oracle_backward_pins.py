"""Pins of the oracle's reverse-mode derivative (CPU only).

The pages state that training runs in chunks ("Kimi K3, explained", "How is KDA trained
efficiently if it is a recurrence?") but print no gradient equations, so ``oracle.backward`` is
the derivative of the recurrence ("The math") taken by hand.  It is pinned to things that do not
share its code:
  every input coordinate against central differences of the forward oracle (a dropped term, a
  wrong sign or a transposed operand anywhere shows up in some coordinate);
  closed forms for a state that neither decays nor is written (beta = 0, alpha = 1);
  the page's overwrite example: a value that a later write under the same key replaces gets
  no gradient.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.timeout(300)


def _case(rng, lengths, H, dk, dv, head_gate=False):
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    N = len(lengths)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = -0.3 * np.log1p(np.exp(rng.standard_normal((T, H) if head_gate else (T, H, dk))))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    s0 = 0.5 * rng.standard_normal((N, H, dk, dv))
    d_o = rng.standard_normal((T, H, dv))
    d_sT = rng.standard_normal((N, H, dk, dv))
    return dict(q=q, k=k, v=v, g=g, beta=b, s0=s0), cu, d_o, d_sT


def _loss(x, cu, d_o, d_sT):
    o, sT = oracle.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, x["s0"], threads=1)
    return float(np.sum(o * d_o) + np.sum(sT * d_sT))


@pytest.mark.parametrize("head_gate", [False, True])
def test_backward_matches_central_differences(head_gate):
    """Mathematics: dL/dx_i = (L(x + h e_i) - L(x - h e_i)) / 2h + O(h^2), for every coordinate of
    every input, with L = <dO, o> + <dS_T, S_T>, two packed sequences (one longer than the
    oracle's 64-token recompute block), two heads and a non-zero initial state."""
    rng = np.random.default_rng(7 + head_gate)
    x, cu, d_o, d_sT = _case(rng, [70, 3], H=2, dk=3, dv=2, head_gate=head_gate)
    dq, dk, dv, dg, db, ds0 = oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, x["s0"],
                                              d_o=d_o, d_sT=d_sT, threads=1)
    grads = dict(q=dq, k=dk, v=dv, g=dg, beta=db, s0=ds0)
    h = 1e-6
    for name, gr in grads.items():
        assert gr.shape == x[name].shape, name
        flat = x[name].reshape(-1)
        for i in range(flat.size):
            keep = flat[i]
            flat[i] = keep + h
            lp = _loss(x, cu, d_o, d_sT)
            flat[i] = keep - h
            lm = _loss(x, cu, d_o, d_sT)
            flat[i] = keep
            fd = (lp - lm) / (2 * h)
            an = gr.reshape(-1)[i]
            assert abs(fd - an) <= 2e-6 * max(1.0, abs(an)), f"d{name}[{i}]: analytic {an}, differences {fd}"


def test_backward_closed_form_no_write_no_decay():
    """beta = 0, alpha = 1: S_t = S_0 for every t and o_t = S_0^T q_t.  With R_t = dS_T +
    sum_{s >= t} q_s do_s^T (the gradient reaching S_t): dq_t = S_0 do_t, dk = dv = 0,
    dbeta_t = (v_t - S_0^T k_t) . (R_t^T k_t), dg_t = rowsum(R_t * S_0), dS_0 = R_1."""
    rng = np.random.default_rng(3)
    T, dk, dv = 9, 5, 4
    q, k, v = rng.standard_normal((T, dk)), rng.standard_normal((T, dk)), rng.standard_normal((T, dv))
    S0, d_o, d_sT = rng.standard_normal((dk, dv)), rng.standard_normal((T, dv)), rng.standard_normal((dk, dv))
    dq, dk_, dv_, dg, db, ds0 = oracle.backward(q[:, None], k[:, None], v[:, None], np.zeros((T, 1, dk)),
                                                np.zeros((T, 1)), None, S0[None, None], d_o=d_o[:, None],
                                                d_sT=d_sT[None, None], threads=1)
    R = d_sT.copy()
    for t in range(T - 1, -1, -1):
        R = R + np.outer(q[t], d_o[t])
        np.testing.assert_allclose(dq[t, 0], S0 @ d_o[t], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(db[t, 0], (v[t] - S0.T @ k[t]) @ (R.T @ k[t]), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dg[t, 0], np.sum(R * S0, axis=1), rtol=1e-12, atol=1e-12)
    assert np.all(dk_ == 0) and np.all(dv_ == 0)
    np.testing.assert_allclose(ds0[0, 0], R, rtol=1e-12, atol=1e-12)


def test_backward_overwritten_value_gets_no_gradient():
    """"The delta: overwrite, don't accumulate": with beta = 1, a unit key and no decay, writing
    (k, a) then (k, b) and reading with q = k returns b whatever a was, so dL/da = 0 and
    dL/db = dL/do.  Plain linear attention (S <- S + k v^T) would return a + b and pass the
    gradient to both."""
    rng = np.random.default_rng(5)
    dk, dv = 4, 3
    key = np.eye(dk)[1]
    a, b = rng.standard_normal(dv), rng.standard_normal(dv)
    q = np.stack([np.zeros(dk), key])[:, None]
    k = np.stack([key, key])[:, None]
    v = np.stack([a, b])[:, None]
    d_o = np.stack([np.zeros(dv), rng.standard_normal(dv)])[:, None]
    dq, dk_, dv_, dg, db, ds0 = oracle.backward(q, k, v, np.zeros((2, 1, dk)), np.ones((2, 1)), d_o=d_o, threads=1)
    np.testing.assert_allclose(dv_[0, 0], 0.0, atol=1e-15)
    np.testing.assert_allclose(dv_[1, 0], d_o[1, 0], rtol=1e-15)
    # the state entering the sequence is overwritten under `key` too: no gradient on that row
    np.testing.assert_allclose(ds0[0, 0][1], 0.0, atol=1e-15)
