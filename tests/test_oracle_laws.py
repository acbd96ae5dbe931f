"""Closed forms, limiting cases and reductions that pin the fp64 oracle.

None of these re-types the oracle's own loop.  Each checks a consequence of
the definition that a plausible mistake would break:

* decay only (b = w = 0) -- the state is the product of the decays times S0
  ("Gated DeltaNet" page, "A retention curve you can calculate");
* a = 1, b = 0 holds the state bit for bit; a -> 0 leaves only the rank-one
  write (same page, "Read the limiting cases");
* a one-hot key touches one key row only, with the erase gate scaling the
  old row and the write gate scaling the value (key-axis gates, "Gated
  DeltaNet-2" blog summary, "Core Mechanism"); dk != dv catches a
  transposed state;
* with no erase the recurrence is decayed linear attention, checked by an
  O(T^2) sum over all token pairs;
* with unit keys and b = 1 the key reads back (sum_c w_c k_c^2) v exactly;
* reductions: tied scalar gates give the Gated DeltaNet step, written here
  element by element from its defining property (decay, then a correction
  along the key sized by the rate times the gap between the value and the
  decayed state's prediction for the key);
  per-channel decay with a tied scalar rate gives KDA; a = 1 gives the delta
  rule (gist.science summary, "Technische Samenvatting", section 1);
* splitting a sequence and resuming from the final state equals one call
  (affine composition, "Gated DeltaNet" page, "What makes the architecture
  more than a recurrence").
"""
import math

import numpy as np
import pytest

from oracle.oracle import gdn2_forward


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_case(seed, B=2, T=23, H=3, dk=5, dv=7, per_key=True, s0=True):
    r = _rng(seed)
    gk = (B, T, H, dk) if per_key else (B, T, H)
    return dict(
        q=r.normal(size=(B, T, H, dk)),
        k=_unit(r.normal(size=(B, T, H, dk))),
        v=r.normal(size=(B, T, H, dv)),
        log_decay=-np.log1p(np.exp(r.normal(-2.0, 1.0, size=gk))),
        erase=1.0 / (1.0 + np.exp(-r.normal(size=gk))),
        write=1.0 / (1.0 + np.exp(-r.normal(size=gk))),
        S0=r.normal(0, 0.5, size=(B, H, dk, dv)) if s0 else None,
    )


def test_decay_only_is_product_of_decays():
    c = _rand_case(1)
    zero = np.zeros_like(c["erase"])
    o, S = gdn2_forward(c["q"], c["k"], c["v"], c["log_decay"], zero, zero, c["S0"])
    G = np.sum(c["log_decay"], axis=1)  # [B,H,dk]
    np.testing.assert_allclose(S, np.exp(G)[..., None] * c["S0"], rtol=1e-13, atol=0)


def test_hold_is_bitwise_and_zero_decay_keeps_only_the_write():
    c = _rand_case(2)
    zero = np.zeros_like(c["erase"])
    o, S = gdn2_forward(c["q"], c["k"], c["v"], zero, zero, zero, c["S0"])
    assert np.array_equal(S, c["S0"])
    # a -> 0: exp(-1000) is 0 in fp64, the old state is gone
    la = np.full_like(c["log_decay"], -1000.0)
    o, S = gdn2_forward(c["q"], c["k"], c["v"], la, c["erase"], c["write"], c["S0"])
    u_last = c["write"][:, -1] * c["k"][:, -1]  # [B,H,dk]
    expect = u_last[..., :, None] * c["v"][:, -1][..., None, :]
    np.testing.assert_allclose(S, expect, rtol=1e-14, atol=1e-15)


def test_one_hot_key_law():
    r = _rng(3)
    T, dk, dv = 9, 4, 6
    S0 = r.normal(size=(1, 1, dk, dv))
    idx = r.integers(0, dk, size=T)
    k = np.zeros((1, T, 1, dk))
    k[0, np.arange(T), 0, idx] = 1.0
    la = -r.uniform(0.0, 1.0, size=(1, T, 1, dk))
    b = r.uniform(size=(1, T, 1, dk))
    w = r.uniform(size=(1, T, 1, dk))
    v = r.normal(size=(1, T, 1, dv))
    q = r.normal(size=(1, T, 1, dk))
    o, S = gdn2_forward(q, k, v, la, b, w, S0)
    ref = S0[0, 0].copy()
    for t in range(T):
        a = np.exp(la[0, t, 0])
        i = idx[t]
        new = a[:, None] * ref
        new[i] = a[i] * (1.0 - b[0, t, 0, i]) * ref[i] + w[0, t, 0, i] * v[0, t, 0]
        ref = new
    np.testing.assert_allclose(S[0, 0], ref, rtol=1e-13, atol=1e-14)


def test_no_erase_is_decayed_linear_attention():
    c = _rand_case(4, T=17)
    zero = np.zeros_like(c["erase"])
    o, S = gdn2_forward(c["q"], c["k"], c["v"], c["log_decay"], zero, c["write"], c["S0"])
    G = np.cumsum(c["log_decay"], axis=1)  # inclusive, [B,T,H,dk]
    B, T, H, dk = c["k"].shape
    o_ref = np.zeros_like(o)
    for t in range(T):
        # initial state seen through the decay up to t
        o_ref[:, t] = np.einsum("bhc,bhcv->bhv", c["q"][:, t] * np.exp(G[:, t]), c["S0"])
        for s in range(t + 1):
            coef = np.sum(c["q"][:, t] * c["write"][:, s] * c["k"][:, s]
                          * np.exp(G[:, t] - G[:, s]), axis=-1)  # [B,H]
            o_ref[:, t] += coef[..., None] * c["v"][:, s]
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    S_ref = np.exp(G[:, -1])[..., None] * c["S0"]
    for s in range(T):
        f = np.exp(G[:, -1] - G[:, s]) * c["write"][:, s] * c["k"][:, s]
        S_ref += f[..., :, None] * c["v"][:, s][..., None, :]
    np.testing.assert_allclose(S, S_ref, rtol=1e-11, atol=1e-12)


def test_full_erase_reads_back_the_written_value():
    c = _rand_case(5)
    ones = np.ones_like(c["erase"])
    # query with the key itself: o_t = S_t^T k_t
    o, S = gdn2_forward(c["k"], c["k"], c["v"], c["log_decay"], ones, c["write"], c["S0"])
    gain = np.sum(c["write"] * c["k"] ** 2, axis=-1)  # [B,T,H]
    np.testing.assert_allclose(o, gain[..., None] * c["v"], rtol=1e-11, atol=1e-12)


def _gdn_reference(q, k, v, alpha_log, beta, S0):
    """Gated DeltaNet / KDA / the delta rule from their defining property,
    element by element: the new state is the decayed old one plus a
    correction along the key, sized by beta times the gap between the value
    and what the decayed state predicts for the key,
        S'[c, j] = a_c S[c, j] + beta k_c (v_j - sum_i a_i k_i S[i, j]),
    and the output reads the new state with the query, o_j = sum_c q_c S'[c, j].
    ``alpha_log`` is [B,T,H] (one decay per head) or [B,T,H,dk] (one per key
    channel).  Plain loops over every index: an independent spelling of the
    update, not the oracle's operation order."""
    B, T, H, dk = k.shape
    dv = v.shape[3]
    S = S0.copy()
    o = np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            st = S[b, h]
            for t in range(T):
                a = [math.exp(alpha_log[b, t, h, c] if alpha_log.ndim == 4 else alpha_log[b, t, h])
                     for c in range(dk)]
                kk, qq, vv, bt = k[b, t, h], q[b, t, h], v[b, t, h], beta[b, t, h]
                pred = [sum(a[i] * kk[i] * st[i, j] for i in range(dk)) for j in range(dv)]
                new = np.empty((dk, dv))
                for c in range(dk):
                    for j in range(dv):
                        new[c, j] = a[c] * st[c, j] + bt * kk[c] * (vv[j] - pred[j])
                st = new
                for j in range(dv):
                    o[b, t, h, j] = sum(qq[c] * st[c, j] for c in range(dk))
            S[b, h] = st
    return o, S


@pytest.mark.parametrize("mode", ["gated_deltanet", "kda", "delta_rule"])
def test_reductions(mode):
    c = _rand_case(6, per_key=True)
    B, T, H, dk = c["k"].shape
    r = _rng(7)
    beta = r.uniform(size=(B, T, H))
    if mode == "gated_deltanet":
        la = -r.uniform(0, 0.5, size=(B, T, H))
    elif mode == "kda":
        la = c["log_decay"]
    else:
        la = np.zeros((B, T, H))
    o_ref, S_ref = _gdn_reference(c["q"], c["k"], c["v"], la, beta, c["S0"])
    # GDN-2 with tied scalar gates (write=None)
    o, S = gdn2_forward(c["q"], c["k"], c["v"], la, beta, None, c["S0"])
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-13)
    # the same with the rate given as equal-entry per-channel erase and write gates
    bvec = np.repeat(beta[..., None], dk, axis=-1)
    o2, S2 = gdn2_forward(c["q"], c["k"], c["v"], la, bvec, bvec.copy(), c["S0"])
    np.testing.assert_allclose(o2, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S2, S_ref, rtol=1e-12, atol=1e-13)


def test_untied_gates_differ_from_tied():
    c = _rand_case(8)
    o1, S1 = gdn2_forward(c["q"], c["k"], c["v"], c["log_decay"], c["erase"], c["write"], c["S0"])
    o2, S2 = gdn2_forward(c["q"], c["k"], c["v"], c["log_decay"], c["erase"], None, c["S0"])
    assert np.max(np.abs(S1 - S2)) > 1e-3


def test_split_and_resume_equals_one_call():
    c = _rand_case(9, T=30)
    args = ("q", "k", "v", "log_decay", "erase", "write")
    o, S = gdn2_forward(*(c[a] for a in args), c["S0"])
    t1 = 11
    oa, Sa = gdn2_forward(*(c[a][:, :t1] for a in args), c["S0"])
    ob, Sb = gdn2_forward(*(c[a][:, t1:] for a in args), Sa)
    assert np.array_equal(np.concatenate([oa, ob], axis=1), o)
    assert np.array_equal(Sb, S)


def test_empty_sequence_returns_initial_state():
    c = _rand_case(10, T=0)
    o, S = gdn2_forward(c["q"], c["k"], c["v"], c["log_decay"], c["erase"], c["write"], c["S0"])
    assert o.shape[1] == 0
    assert np.array_equal(S, c["S0"])


def test_q_scale_is_linear():
    c = _rand_case(11)
    args = ("q", "k", "v", "log_decay", "erase", "write")
    o1, S1 = gdn2_forward(*(c[a] for a in args), c["S0"])
    o2, S2 = gdn2_forward(*(c[a] for a in args), c["S0"], q_scale=0.25)
    np.testing.assert_allclose(o2, 0.25 * o1, rtol=1e-14, atol=0)
    assert np.array_equal(S1, S2)
