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

The value-write form and the raw-input preparation are pinned the same way
(finite differences), and further: the value-write forward to the C oracle's;
with one erase and one write gate per head the two forms are the same
operation, so their gradients must agree; the torch input preparation to the
numpy one (itself pinned to scipy); and the raw-input gradients to the
prepared-input gradients through the chain rule of -softplus, sigmoid and the
L2 normalisation written out by hand.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle.oracle import gdn2_forward, prepare_inputs
from oracle.oracle_bwd import gdn2_backward, prepare, recurrence


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


def _loss(inp, d_o, d_state, q_scale, value_write=False, raw=False):
    """L = <d_o, o> + <d_state, S_T> evaluated with the differentiable forward
    (``raw``: the gate entries are logits and q, k are normalised first)."""
    t = lambda x: None if x is None else torch.as_tensor(np.asarray(x, dtype=np.float64))
    q, k, la, b, w = t(inp["q"]), t(inp["k"]), t(inp["log_decay"]), t(inp["erase"]), t(inp["write"])
    if raw:
        q, k, la, b, w = prepare(q, k, la, b, w)
    o, S = recurrence(q, k, t(inp["v"]), la, b, w, t(inp["S0"]), q_scale, value_write)
    return float((o.numpy() * d_o).sum() + (S.numpy() * d_state).sum())


def _fd_check(inp, g, d_o, d_state, qs, names, **kw):
    h = 1e-6
    for key, gkey in names:
        x = inp[key]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(inp, d_o, d_state, qs, **kw)
            x[idx] = old - h
            lm = _loss(inp, d_o, d_state, qs, **kw)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g[gkey], fd, rtol=1e-6, atol=1e-8, err_msg=key)


NAMES = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_decay", "d_log_decay"), ("erase", "d_erase"),
         ("S0", "d_state0"), ("write", "d_write")]


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
    _fd_check(inp, g, d_o, d_state, qs, NAMES[:6] + ([] if tied else NAMES[6:]))


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


def _vw_case(r, gates, B=1, T=4, H=2, dk=3, dv=2):
    """A value-write case: the write gate per value channel (or per head)."""
    inp = _case(r, B, T, H, dk, dv, gates=gates)
    ws = (B, T, H, dv) if gates == "key" else (B, T, H)
    inp["write"] = 1 / (1 + np.exp(-r.standard_normal(ws)))
    return inp


def test_value_write_forward_matches_c_oracle():
    r = np.random.default_rng(21)
    inp = _vw_case(r, "key", B=2, T=7, H=2, dk=5, dv=4)
    t = lambda x: torch.as_tensor(np.asarray(x, dtype=np.float64))
    o_t, S_t = recurrence(*[t(inp[n]) for n in ("q", "k", "v", "log_decay", "erase", "write", "S0")],
                          q_scale=1.0, value_write=True)
    o_c, S_c = gdn2_forward(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"],
                            inp["S0"], value_write=True)
    np.testing.assert_allclose(o_t.numpy(), o_c, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S_t.numpy(), S_c, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("gates", ["key", "head"])
def test_value_write_gradients_match_finite_differences(gates):
    r = np.random.default_rng(22)
    inp = _vw_case(r, gates)
    qs = 0.8
    d_o, d_state = r.standard_normal(inp["v"].shape), r.standard_normal(inp["S0"].shape)
    g = gdn2_backward(**inp, d_o=d_o, d_state=d_state, q_scale=qs, value_write=True)
    _fd_check(inp, g, d_o, d_state, qs, NAMES, value_write=True)


def test_forms_agree_with_scalar_gates():
    # one erase and one write gate per head: (I - k (b k)^T) Sbar + k (w v)^T
    # is Sbar - (b k)(k^T Sbar) + (w k) v^T, so every gradient is the same
    r = np.random.default_rng(23)
    inp = _case(r, B=2, T=6, H=2, dk=4, dv=3, gates="head")
    d_o, d_state = r.standard_normal(inp["v"].shape), r.standard_normal(inp["S0"].shape)
    gk = gdn2_backward(**inp, d_o=d_o, d_state=d_state, q_scale=1.1)
    gv = gdn2_backward(**inp, d_o=d_o, d_state=d_state, q_scale=1.1, value_write=True)
    for key in ("dq", "dk", "dv", "d_log_decay", "d_erase", "d_write", "d_state0"):
        np.testing.assert_allclose(gv[key], gk[key], rtol=1e-11, atol=1e-12, err_msg=key)


def _raw_case(r, gates="key", B=1, T=4, H=2, dk=3, dv=2):
    gs = (B, T, H, dk) if gates == "key" else (B, T, H)
    return dict(q=r.standard_normal((B, T, H, dk)) * 2, k=r.standard_normal((B, T, H, dk)) * 0.7,
                v=r.standard_normal((B, T, H, dv)), log_decay=r.standard_normal(gs) - 1.0,
                erase=r.standard_normal(gs), write=r.standard_normal(gs),
                S0=r.standard_normal((B, H, dk, dv)) * 0.5)


def test_torch_preparation_matches_numpy():
    r = np.random.default_rng(24)
    inp = _raw_case(r, B=2, T=5, H=2, dk=6)
    inp["q"][0, 1, 1] = 0.0  # a zero row stays zero
    t = lambda x: torch.as_tensor(np.asarray(x, dtype=np.float64))
    got = prepare(t(inp["q"]), t(inp["k"]), t(inp["log_decay"]), t(inp["erase"]), t(inp["write"]))
    want = prepare_inputs(inp["q"], inp["k"], inp["log_decay"], inp["erase"], inp["write"])
    for a, b in zip(got, want):
        np.testing.assert_allclose(a.numpy(), b, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("gates,vw", [("key", False), ("head", False), ("key", True)])
def test_raw_input_gradients_match_finite_differences(gates, vw):
    r = np.random.default_rng(25)
    inp = _raw_case(r, gates)
    if vw:
        inp["write"] = r.standard_normal(inp["v"].shape if gates == "key" else inp["v"].shape[:3])
    qs = 0.9
    d_o, d_state = r.standard_normal(inp["v"].shape), r.standard_normal(inp["S0"].shape)
    g = gdn2_backward(**inp, d_o=d_o, d_state=d_state, q_scale=qs, raw=True, value_write=vw)
    _fd_check(inp, g, d_o, d_state, qs, NAMES, raw=True, value_write=vw)


def test_raw_gradients_by_the_chain_rule():
    # d/dx (-softplus x) = -sigmoid x, d/dx sigmoid x = s (1 - s), and for
    # n = x / |x|: dx = (dn - n (n . dn)) / |x|
    r = np.random.default_rng(26)
    raw = _raw_case(r, "key", B=2, T=5, H=2, dk=4, dv=3)
    d_o, d_state = r.standard_normal(raw["v"].shape), r.standard_normal(raw["S0"].shape)
    g_raw = gdn2_backward(**raw, d_o=d_o, d_state=d_state, raw=True)
    q, k, la, b, w = prepare_inputs(raw["q"], raw["k"], raw["log_decay"], raw["erase"], raw["write"])
    g = gdn2_backward(q, k, raw["v"], la, b, w, raw["S0"], d_o=d_o, d_state=d_state)
    sig = lambda x: 1 / (1 + np.exp(-x))
    np.testing.assert_allclose(g_raw["d_log_decay"], -sig(raw["log_decay"]) * g["d_log_decay"], rtol=1e-10,
                               atol=1e-12)
    for key, x in (("d_erase", raw["erase"]), ("d_write", raw["write"])):
        np.testing.assert_allclose(g_raw[key], sig(x) * (1 - sig(x)) * g[key], rtol=1e-10, atol=1e-12)
    for key, x, n in (("dq", raw["q"], q), ("dk", raw["k"], k)):
        dn = g[key]
        want = (dn - n * (n * dn).sum(-1, keepdims=True)) / np.linalg.norm(x, axis=-1, keepdims=True)
        np.testing.assert_allclose(g_raw[key], want, rtol=1e-10, atol=1e-12)
    for key in ("dv", "d_state0"):
        np.testing.assert_allclose(g_raw[key], g[key], rtol=1e-12, atol=1e-12)


# ---- the hand-written reverse pass of the C oracle (gdn2_backward_c) -------
# It serves the full-size GPU gradient checks, where autograd's tape would be
# too slow and too large.  It is pinned to central finite differences of the
# C forward (a different program from the one it differentiates by hand) and
# to the autograd gradients above, for every gate kind, tied and untied, with
# segment boundaries of its checkpointed recomputation inside the sequence.

def _c_loss(inp, d_o, d_state, qs):
    o, S = gdn2_forward(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"],
                        inp["S0"], q_scale=qs, threads=1)
    return float((o * d_o).sum() + (S * d_state).sum())


@pytest.mark.parametrize("gates,tied", [("key", False), ("head", False), ("key", True), ("head", True)])
def test_c_reverse_pass_equals_finite_differences_of_the_c_forward(gates, tied):
    from oracle.oracle import gdn2_backward_c

    r = np.random.Generator(np.random.PCG64(900 + 2 * tied + (gates == "head")))
    inp = _case(r, B=1, T=5, H=2, dk=3, dv=2, gates=gates, tied=tied)
    d_o = r.standard_normal((1, 5, 2, 2))
    d_state = r.standard_normal((1, 2, 3, 2))
    qs = 0.8
    g = gdn2_backward_c(**inp, d_o=d_o, d_state=d_state, q_scale=qs, threads=1)
    names = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_decay", "d_log_decay"), ("erase", "d_erase"),
             ("S0", "d_state0")] + ([] if tied else [("write", "d_write")])
    h = 1e-6
    for key, gkey in names:
        x = inp[key]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _c_loss(inp, d_o, d_state, qs)
            x[idx] = old - h
            lm = _c_loss(inp, d_o, d_state, qs)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g[gkey], fd, rtol=1e-6, atol=1e-7, err_msg=gkey)


@pytest.mark.parametrize("gates,tied,T", [("key", False, 150), ("head", False, 64), ("key", True, 129),
                                          ("head", True, 1)])
def test_c_reverse_pass_equals_autograd(gates, tied, T):
    from oracle.oracle import gdn2_backward_c

    r = np.random.Generator(np.random.PCG64(950 + T))
    inp = _case(r, B=2, T=T, H=2, dk=6, dv=5, gates=gates, tied=tied)
    d_o = r.standard_normal((2, T, 2, 5))
    d_state = r.standard_normal((2, 2, 6, 5))
    a = gdn2_backward(**inp, d_o=d_o, d_state=d_state, q_scale=0.6)
    c = gdn2_backward_c(**inp, d_o=d_o, d_state=d_state, q_scale=0.6, threads=2)
    for n in ("dq", "dk", "dv", "d_log_decay", "d_erase", "d_write", "d_state0"):
        if a[n] is None:
            assert c[n] is None
            continue
        np.testing.assert_allclose(c[n], a[n], rtol=1e-10, atol=1e-12, err_msg=n)
    # no cotangent of o, no initial state: only the final state's gradient flows
    inp["S0"] = None
    a = gdn2_backward(**inp, d_o=None, d_state=d_state)
    c = gdn2_backward_c(**inp, d_o=None, d_state=d_state)
    for n in ("dq", "dk", "dv", "d_log_decay", "d_erase", "d_state0"):
        np.testing.assert_allclose(c[n], a[n], rtol=1e-10, atol=1e-12, err_msg=n)
