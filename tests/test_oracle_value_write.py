"""Pins of the oracle's value-write form.

The gist.science summary ("Methodologie", 1. "Gated Delta-regel-2") writes
the update as S_t = (I - k_t (b_t .* k_t)^T) D_t S_{t-1} + k_t (w_t .* v_t)^T:
the erase gate b (per key channel) weights the read of the decayed state,
the erase and the write both run along k, and the write gate w has one
factor per VALUE channel.  The pages print no numbers for it, so the pins
are a case worked by hand from that equation, the reduction the same
summary states (gates tied to one scalar give back KDA, i.e. the key-axis
form), and the no-erase closed form.
"""
import math

import numpy as np
import pytest

from oracle.oracle import gdn2_forward


def _one(S0, k, v, q, alpha, b, w, form):
    f = lambda x: np.asarray(x, dtype=np.float64).reshape(1, 1, 1, -1)
    return gdn2_forward(f(q), f(k), f(v), np.full((1, 1, 1), math.log(alpha)), f(b), f(w),
                        np.asarray(S0, dtype=np.float64).reshape(1, 1, 2, 2), threads=1,
                        value_write=form)


def test_worked_by_hand():
    # Sbar = 0.8 S0 = [[1.6, 2.4], [4.0, 0.8]]; b.*k = [0.3, 0.8];
    # m = Sbar^T (b.*k) = [3.68, 1.36]; Sbar - k m^T = [[-0.608, 1.584], [1.056, -0.288]];
    # k (w.*v)^T = [0.6, 0.8]^T [9, 4.5] = [[5.4, 2.7], [7.2, 3.6]]
    S0 = [[2.0, 3.0], [5.0, 1.0]]
    o, S = _one(S0, [0.6, 0.8], [9.0, 9.0], [1.0, 0.0], 0.8, [0.5, 1.0], [1.0, 0.5], True)
    np.testing.assert_allclose(S[0, 0], [[4.792, 4.284], [8.256, 3.312]], atol=1e-12)
    np.testing.assert_allclose(o[0, 0, 0], [4.792, 4.284], atol=1e-12)
    # the key-axis form on the same numbers differs (erase (b.*k) m^T, write (w.*k) v^T)
    o2, S2 = _one(S0, [0.6, 0.8], [9.0, 9.0], [1.0, 0.0], 0.8, [0.5, 1.0], [1.0, 0.5], False)
    np.testing.assert_allclose(S2[0, 0], [[5.752, 7.176], [4.272, 2.736]], atol=1e-12)


@pytest.mark.parametrize("tied_scalar", [True, False])
def test_scalar_gates_give_the_key_axis_form(tied_scalar):
    r = np.random.default_rng(21)
    B, T, H, dk, dv = 2, 17, 2, 5, 3
    q, k = r.standard_normal((B, T, H, dk)), r.standard_normal((B, T, H, dk)) * 0.5
    v = r.standard_normal((B, T, H, dv))
    la = -np.logaddexp(0, r.standard_normal((B, T, H, dk)))
    b = 1 / (1 + np.exp(-r.standard_normal((B, T, H))))
    w = b.copy() if tied_scalar else 1 / (1 + np.exp(-r.standard_normal((B, T, H))))
    S0 = r.standard_normal((B, H, dk, dv))
    o1, S1 = gdn2_forward(q, k, v, la, b, w, S0, threads=1, value_write=True)
    o0, S0_ = gdn2_forward(q, k, v, la, b, w, S0, threads=1)
    np.testing.assert_allclose(o1, o0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S1, S0_, rtol=1e-12, atol=1e-12)


def test_no_erase_is_a_gated_write():
    r = np.random.default_rng(22)
    dk, dv = 4, 6
    S0 = r.standard_normal((1, 1, dk, dv))
    k, q = r.standard_normal(dk), r.standard_normal(dk)
    v, w = r.standard_normal(dv), r.uniform(size=dv)
    la = -r.uniform(0, 1, size=dk)
    f = lambda x: x.reshape(1, 1, 1, -1)
    o, S = gdn2_forward(f(q), f(k), f(v), f(la), np.zeros((1, 1, 1, dk)), f(w), S0, threads=1,
                        value_write=True)
    want = np.exp(la)[:, None] * S0[0, 0] + np.outer(k, w * v)
    np.testing.assert_allclose(S[0, 0], want, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o[0, 0, 0], want.T @ q, rtol=1e-13, atol=1e-13)


def test_needs_a_write_gate():
    z = np.zeros((1, 1, 1, 2))
    with pytest.raises(ValueError):
        gdn2_forward(z, z, z, z, z, None, None, value_write=True)
