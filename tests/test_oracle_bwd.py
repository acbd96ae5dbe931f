"""Pins of the gradient oracle (oracle/oracle_bwd.py).

The gradients come from torch.autograd over the token recurrence, so two
things can be wrong: the differentiable forward, and what is asked of
autograd.  The forward is pinned to the pages' worked examples (the same
fixtures as the C oracle's pins) and to the C oracle; the gradients are
pinned to central finite differences of that forward and to closed forms of
special cases that follow from the recurrence by hand:

* hold (a = 1, b = w = 0): the state never changes, so with
  G_t = q_scale sum_{tau >= t} q_tau dO_tau^T + dS_T (the gradient flowing
  into S_t), dq_t = q_scale S0 dO_t, dS0 = G_0, dv = dk = 0,
  d log a_t[c] = sum_j G_t[c,j] S0[c,j], dw_t[c] = k_t[c] (G_t v_t)[c],
  db_t[c] = -k_t[c] (G_t m_t)[c] with m_t = S0^T k_t;
* decay only (b = w = 0): S_tau = Diag(exp(g_tau)) S0 with g the running sum
  of log a, so d log a_t[c] = sum_{tau >= t} q_scale q_tau[c] exp(g_tau[c])
  (S0[c,:] . dO_tau) + exp(g_T[c]) (S0[c,:] . dS_T[c,:]);
* one token: o = S_1^T (s q) and S_1 is linear in v with coefficient u, so
  dv = (s q . u) dO + dS_1^T u.
A dropped term, a wrong sign, a transposed operand or a gradient taken
against the stale state fails one of these.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle.oracle import gdn2_forward
from oracle.oracle_bwd import gdn2_backward, recurrence


def _rand(shape, r, lo=None):
    return r.standard_normal(shape)


def _case(r, B=1, T=4, H=2, dk=3, dv=2, gates="key", tied=False, s0=True):
    gs = (B, T, H, dk) if gates == "key" else (B, T, H)
    return dict(
        q=r.standard_normal((B, T, H, dk)), k=r.standard_normal((B, T, H, dk)) * 0.6,
        v=r.standard_normal((B, T, H, dv)),
        log_decay=-np.logaddexp(0, r.standard_normal(gs) - 1.0),
        erase=1 / (1 + np.exp(-r.standard_normal(gs))),
        write=None if tied else 1 / (1 + np.exp(-r.standard_normal(gs))),
        S0=r.standard_normal((B, H, dk, dv)) * 0.5 if s0 else None)


def _loss(inp, d_o, d_state, q_scale):
    """L = <d_o, o> + <d_state, S_T> evaluated with the differentiable forward."""
    t = lambda x: None if x is None else torch.as_tensor(np.asarray(x, dtype=np.float64))
    o, S = recurrence(t(inp["q"]), t(inp["k"]), t(inp["v"]), t(inp["log_decay"]), t(inp["erase"]),
                      t(inp["write"]), t(inp["S0"]), q_scale)
    return float((o.numpy() * d_o).sum() + (S.numpy() * d_state).sum())


def test_forward_matches_page_examples(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "course_slides_trace.json")))
    f = lambda x: torch.tensor(x, dtype=torch.float64).reshape(1, 1, 1, -1)
    o, S = recurrence(f(g["query"]), f(g["key"]), f(g["value"]),
                      torch.full((1, 1, 1), math.log(g["alpha"]), dtype=torch.float64),
                      torch.full((1, 1, 1), g["beta"], dtype=torch.float64), None,
                      torch.tensor(g["state0"], dtype=torch.float64).reshape(1, 1, 2, 2))
    np.testing.assert_allclose(S[0, 0].numpy(), g["state1"], atol=1e-12)
    np.testing.assert_allclose(o[0, 0, 0].numpy(), g["read_after_update"], atol=1e-12)
    g = json.load(open(os.path.join(golden_dir, "gated_deltanet_scalar_step.json")))
    one = lambda x: torch.tensor([x], dtype=torch.float64).reshape(1, 1, 1, 1)
    o, S = recurrence(one(g["key"]), one(g["key"]), one(g["value"]),
                      torch.full((1, 1, 1), math.log(g["alpha"]), dtype=torch.float64),
                      torch.full((1, 1, 1), g["beta"], dtype=torch.float64), None,
                      one(g["state0"]))
    assert float(S) == pytest.approx(g["expected_state"], abs=1e-12)


@pytest.mark.parametrize("gates,tied", [("key", False), ("head", True), ("head", False)])
def test_forward_matches_c_oracle(gates, tied):
    r = np.random.default_rng(5)
    inp = _case(r, B=2, T=9, H=2, dk=5, dv=4, gates=gates, tied=tied)
    o_c, S_c = gdn2_forward(**inp, q_scale=0.8, threads=1)
    t = lambda x: None if x is None else torch.as_tensor(x)
    o_t, S_t = recurrence(t(inp["q"]), t(inp["k"]), t(inp["v"]), t(inp["log_decay"]),
                          t(inp["erase"]), t(inp["write"]), t(inp["S0"]), 0.8)
    np.testing.assert_allclose(o_t.numpy(), o_c, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S_t.numpy(), S_c, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("gates,tied,s0", [("key", False, True), ("key", True, True),
                                           ("head", False, True), ("head", True, False)])
def test_gradients_match_finite_differences(gates, tied, s0):
    r = np.random.default_rng(11)
    inp = _case(r, gates=gates, tied=tied, s0=s0)
    if inp["S0"] is None:
        inp["S0"] = np.zeros((1, 2, 3, 2))
    qs = 0.7
    d_o = r.standard_normal(inp["v"].shape)
    d_state = r.standard_normal(inp["S0"].shape)
    g = gdn2_backward(**inp, d_o=d_o, d_state=d_state, q_scale=qs)
    names = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_decay", "d_log_decay"),
             ("erase", "d_erase"), ("S0", "d_state0")] + ([] if tied else [("write", "d_write")])
    h = 1e-6
    for key, gkey in names:
        x = inp[key]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(inp, d_o, d_state, qs)
            x[idx] = old - h
            lm = _loss(inp, d_o, d_state, qs)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g[gkey], fd, rtol=1e-6, atol=1e-8, err_msg=key)


def test_hold_closed_form():
    r = np.random.default_rng(12)
    B, T, H, dk, dv, qs = 1, 5, 1, 3, 4, 1.3
    inp = _case(r, B, T, H, dk, dv)
    inp["log_decay"][:] = 0.0
    inp["erase"][:] = 0.0
    inp["write"][:] = 0.0
    d_o, d_state = r.standard_normal((B, T, H, dv)), r.standard_normal((B, H, dk, dv))
    g = gdn2_backward(**inp, d_o=d_o, d_state=d_state, q_scale=qs)
    S0 = inp["S0"][0, 0]
    q, k, v, dO = inp["q"][0, :, 0], inp["k"][0, :, 0], inp["v"][0, :, 0], d_o[0, :, 0]
    Gt = [qs * sum(np.outer(q[u], dO[u]) for u in range(t, T)) + d_state[0, 0] for t in range(T)]
    for t in range(T):
        np.testing.assert_allclose(g["dq"][0, t, 0], qs * S0 @ dO[t], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g["d_log_decay"][0, t, 0], (Gt[t] * S0).sum(1), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(g["d_write"][0, t, 0], k[t] * (Gt[t] @ v[t]), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(g["d_erase"][0, t, 0], -k[t] * (Gt[t] @ (S0.T @ k[t])), rtol=1e-10,
                                   atol=1e-12)
    np.testing.assert_allclose(g["d_state0"][0, 0], Gt[0], rtol=1e-12, atol=1e-12)
    assert np.abs(g["dv"]).max() == 0 and np.abs(g["dk"]).max() == 0


def test_decay_only_closed_form():
    r = np.random.default_rng(13)
    B, T, H, dk, dv, qs = 1, 6, 1, 4, 3, 0.9
    inp = _case(r, B, T, H, dk, dv)
    inp["erase"][:] = 0.0
    inp["write"][:] = 0.0
    d_o, d_state = r.standard_normal((B, T, H, dv)), r.standard_normal((B, H, dk, dv))
    g = gdn2_backward(**inp, d_o=d_o, d_state=d_state, q_scale=qs)
    la, q, S0, dO = inp["log_decay"][0, :, 0], inp["q"][0, :, 0], inp["S0"][0, 0], d_o[0, :, 0]
    gc = np.cumsum(la, 0)
    for t in range(T):
        want = sum(qs * q[u] * np.exp(gc[u]) * (S0 @ dO[u]) for u in range(t, T))
        want = want + np.exp(gc[-1]) * (S0 * d_state[0, 0]).sum(1)
        np.testing.assert_allclose(g["d_log_decay"][0, t, 0], want, rtol=1e-10, atol=1e-12)


def test_one_token_value_gradient():
    r = np.random.default_rng(14)
    qs = 1.7
    inp = _case(r, 1, 1, 1, 4, 3)
    d_o, d_state = r.standard_normal((1, 1, 1, 3)), r.standard_normal((1, 1, 4, 3))
    g = gdn2_backward(**inp, d_o=d_o, d_state=d_state, q_scale=qs)
    u = inp["write"][0, 0, 0] * inp["k"][0, 0, 0]
    want = qs * (inp["q"][0, 0, 0] @ u) * d_o[0, 0, 0] + d_state[0, 0].T @ u
    np.testing.assert_allclose(g["dv"][0, 0, 0], want, rtol=1e-12, atol=1e-12)


def test_no_cotangent_gives_zero_gradients():
    r = np.random.default_rng(15)
    inp = _case(r)
    g = gdn2_backward(**inp)
    for key in ("dq", "dk", "dv", "d_log_decay", "d_erase", "d_write", "d_state0"):
        assert np.abs(g[key]).max() == 0
