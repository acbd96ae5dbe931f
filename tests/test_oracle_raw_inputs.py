"""Pins of the oracle's input preparation (gate logits, q/k normalisation).

The workloads define the gates through their logits (decay a = exp(-softplus
(x)), erase and write sigmoid(x)) and normalise q and k per token-head.  The
oracle's ``prepare_inputs`` is pinned to library routines that compute the
same functions (scipy's ``log_expit`` and ``expit``, numpy's ``norm``), to
the closed forms at x = 0 (a = b = w = 1/2), and to the invariance that
normalisation implies (scaling q or k by a positive factor changes nothing).
"""
import math

import numpy as np
import pytest
from scipy.special import expit, log_expit

from oracle.oracle import gdn2_forward, gdn2_forward_raw, prepare_inputs


def _raw(r, B=2, T=11, H=2, dk=6, dv=5, gates="key", tied=False):
    gs = (B, T, H, dk) if gates == "key" else (B, T, H)
    return dict(q=r.standard_normal((B, T, H, dk)) * 3, k=r.standard_normal((B, T, H, dk)) * 2,
                v=r.standard_normal((B, T, H, dv)), x_decay=r.normal(-2, 1, gs), x_erase=r.standard_normal(gs),
                x_write=None if tied else r.standard_normal(gs), S0=r.standard_normal((B, H, dk, dv)) * 0.1)


@pytest.mark.parametrize("gates,tied", [("key", False), ("head", True)])
def test_matches_library_routines(gates, tied):
    r = np.random.default_rng(31)
    x = _raw(r, gates=gates, tied=tied)
    o, S = gdn2_forward_raw(**x, threads=1)
    nq = x["q"] / np.linalg.norm(x["q"], axis=-1, keepdims=True)
    nk = x["k"] / np.linalg.norm(x["k"], axis=-1, keepdims=True)
    o2, S2 = gdn2_forward(nq, nk, x["v"], log_expit(-x["x_decay"]), expit(x["x_erase"]),
                          None if tied else expit(x["x_write"]), x["S0"], threads=1)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, S2, rtol=1e-12, atol=1e-12)


def test_zero_logits_give_one_half():
    q, k, la, b, w = prepare_inputs(np.ones((1, 1, 1, 4)), np.ones((1, 1, 1, 4)), np.zeros((1, 1, 1)),
                                    np.zeros((1, 1, 1)), np.zeros((1, 1, 1)))
    assert math.exp(la[0, 0, 0]) == pytest.approx(0.5, abs=1e-15)
    assert b[0, 0, 0] == 0.5 and w[0, 0, 0] == 0.5
    np.testing.assert_allclose(q, 0.5, atol=1e-15)  # [1,1,1,1] / 2


def test_normalisation_is_scale_free_and_keeps_zero():
    r = np.random.default_rng(32)
    x = _raw(r)
    o, S = gdn2_forward_raw(**x, threads=1)
    x2 = dict(x, q=x["q"] * 7.5, k=x["k"] * 0.01)
    o2, S2 = gdn2_forward_raw(**x2, threads=1)
    np.testing.assert_allclose(o2, o, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(S2, S, rtol=1e-10, atol=1e-12)
    q, k, *_ = prepare_inputs(np.zeros((1, 1, 1, 3)), np.zeros((1, 1, 1, 3)), np.zeros((1, 1, 1)),
                              np.zeros((1, 1, 1)))
    assert np.all(q == 0) and np.all(k == 0)


def test_without_normalisation_q_k_pass_through():
    r = np.random.default_rng(33)
    x = _raw(r)
    o, _ = gdn2_forward_raw(**x, qk_l2norm=False, threads=1)
    o2, _ = gdn2_forward(x["q"], x["k"], x["v"], -np.logaddexp(0, x["x_decay"]), expit(x["x_erase"]),
                         expit(x["x_write"]), x["S0"], threads=1)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
