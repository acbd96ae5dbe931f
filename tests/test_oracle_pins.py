"""Pins of the fp64 oracle to the numbers the pages print.

Each test feeds the oracle the exact inputs of a worked example on the pages
(fixtures in tests/golden/, each citing its page and section) and checks the
printed result to the printed precision.  A mistake in the oracle's order of
operations (decay after the write), in the read (undecayed state), in a sign,
or in the output read (before the update) fails one of these.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle.oracle import gdn2_forward

pytestmark = pytest.mark.filterwarnings("ignore")


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _one_token(S0, k, v, q, alpha, beta, write=None):
    """Run the oracle for one token of one head with scalar gates."""
    S0 = np.asarray(S0, dtype=np.float64)
    dk, dv = S0.shape
    shp = (1, 1, 1)
    o, S = gdn2_forward(
        np.asarray(q, dtype=np.float64).reshape(shp + (dk,)),
        np.asarray(k, dtype=np.float64).reshape(shp + (dk,)),
        np.asarray(v, dtype=np.float64).reshape(shp + (dv,)),
        np.full(shp, math.log(alpha)),
        np.full(shp, beta),
        None if write is None else np.full(shp, write),
        S0.reshape(1, 1, dk, dv),
        threads=1,
    )
    return o[0, 0, 0], S[0, 0]


def test_scalar_step_decays_before_the_error(golden_dir):
    g = _load(golden_dir, "gated_deltanet_scalar_step.json")
    o, S = _one_token([[g["state0"]]], [g["key"]], [g["value"]], [g["key"]],
                      g["alpha"], g["beta"])
    assert S[0, 0] == pytest.approx(g["expected_state"], abs=1e-12)
    assert abs(S[0, 0] - g["stale_error_variant_state"]) > 0.4
    # the query read sees the updated state
    assert o[0] == pytest.approx(g["expected_state"], abs=1e-12)


def test_two_by_two_trace(golden_dir):
    g = _load(golden_dir, "course_slides_trace.json")
    tol = 0.5 * 10 ** -g["printed_decimals"]
    o, S1 = _one_token(g["state0"], g["key"], g["value"], g["query"], g["alpha"], g["beta"])
    np.testing.assert_allclose(S1, g["state1"], atol=tol, rtol=0)
    np.testing.assert_allclose(S1, g["state1"], atol=1e-12, rtol=0)  # exact for these inputs
    np.testing.assert_allclose(o, g["read_after_update"], atol=1e-12)
    # residual error after one partial correction is exactly (1 - beta) * e
    k = np.asarray(g["key"])
    resid = np.asarray(g["value"]) - S1.T @ k
    np.testing.assert_allclose(resid, g["residual_error"], atol=1e-12)
    np.testing.assert_allclose(resid, (1 - g["beta"]) * np.asarray(g["error"]), atol=1e-12)
    # the reversed order (correct, then decay) is a different model
    assert np.max(np.abs(S1 - np.asarray(g["reversed_order_state"]))) > 0.8


def test_two_by_two_beta_extremes(golden_dir):
    g = _load(golden_dir, "course_slides_trace.json")
    _, S_b0 = _one_token(g["state0"], g["key"], g["value"], g["query"], g["alpha"], 0.0)
    np.testing.assert_allclose(S_b0, g["beta0_state"], atol=1e-12)
    _, S_b1 = _one_token(g["state0"], g["key"], g["value"], g["query"], g["alpha"], 1.0)
    np.testing.assert_allclose(S_b1[0], g["beta1_row0"], atol=1e-12)
    # k = [1, 0] does not select row 2: it is only decayed
    np.testing.assert_allclose(S_b1[1], g["decayed_state"][1], atol=1e-12)


def test_two_by_two_decay_only(golden_dir):
    g = _load(golden_dir, "course_slides_trace.json")
    S0 = np.asarray(g["state0"], dtype=np.float64)
    T = 2
    o, S = gdn2_forward(np.zeros((1, T, 1, 2)), np.zeros((1, T, 1, 2)), np.zeros((1, T, 1, 2)),
                        np.full((1, T, 1), math.log(g["alpha"])), np.zeros((1, T, 1)), None,
                        S0.reshape(1, 1, 2, 2), threads=1)
    np.testing.assert_allclose(S[0, 0], g["decay_only_two_steps"], atol=1e-12)


def _retention(alpha, steps, per_key=False):
    """Decay-only run of a 1x1 state holding 1.0; returns the trace."""
    T = steps
    shape = (1, T, 1, 1) if per_key else (1, T, 1)
    o, S = gdn2_forward(np.ones((1, T, 1, 1)), np.zeros((1, T, 1, 1)), np.zeros((1, T, 1, 1)),
                        np.full(shape, math.log(alpha)), np.zeros(shape), None,
                        np.ones((1, 1, 1, 1)), threads=1)
    return o[0, :, 0, 0], S[0, 0, 0, 0]


def test_decay_trace_and_threshold(golden_dir):
    g = _load(golden_dir, "course_slides_trace.json")
    trace, _ = _retention(g["alpha"], 12)
    full = np.concatenate([[1.0], trace])
    np.testing.assert_allclose(full[:4], g["decay_only_trace"], atol=1e-12)
    first_below = int(np.argmax(full < 0.1))
    assert first_below == g["first_step_below_0p1"]
    assert full[first_below] == pytest.approx(g["value_at_11"], abs=5e-4)


def test_half_lives_and_retention(golden_dir):
    g = _load(golden_dir, "half_lives.json")
    for r in g["retention"]:
        trace, _ = _retention(r["alpha"], r["steps"])
        assert trace[-1] == pytest.approx(r["value"], abs=0.5 * 10 ** -r["decimals"])
    for h in g["half_life"]:
        hl = math.log(0.5) / math.log(h["alpha"])
        assert hl == pytest.approx(h["value"], abs=0.5 * 10 ** -h["decimals"] + 1e-12)
        # the oracle's retention crosses one half between floor and ceil of it
        n = int(math.ceil(hl)) + 1
        trace, _ = _retention(h["alpha"], n, per_key=True)
        full = np.concatenate([[1.0], trace])
        lo, hi = int(math.floor(hl)), int(math.ceil(hl))
        assert full[lo] >= 0.5 - 1e-12 and full[hi] <= 0.5 + 1e-12
    for gr in g["growth"]:
        trace, _ = _retention(gr["alpha"], gr["steps"])
        assert trace[-1] == pytest.approx(gr["value"], abs=0.5 * 10 ** -gr["decimals"])
    a2k = g["alpha_for_half_at_2000"]
    alpha = 0.5 ** (1.0 / a2k["steps"])
    assert alpha == pytest.approx(a2k["alpha"], abs=0.5 * 10 ** -a2k["decimals"])
    trace, _ = _retention(alpha, a2k["steps"])
    assert trace[-1] == pytest.approx(0.5, abs=1e-12)
