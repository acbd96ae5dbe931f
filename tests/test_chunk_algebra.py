"""The chunkwise (WY/UT) form equals the token recurrence on small inputs.

This is the "chunked versus sequential" check on the CPU, in fp64: the
helper in tests/chunk_algebra.py (the algebra the GPU kernels implement)
against the oracle, for several chunk lengths, a ragged last chunk, every
gate kind, tied and untied gates, zero and nonzero initial state.  Chunk
length 1 is the recurrence itself.
"""
import numpy as np
import pytest

from oracle.oracle import gdn2_forward
from tests.chunk_algebra import chunk_forward


def _case(seed, B=1, T=37, H=2, dk=6, dv=5, gates="key", s0=True, spike=False):
    r = np.random.Generator(np.random.PCG64(seed))
    gs = (B, T, H, dk) if gates == "key" else (B, T, H)
    k = r.normal(size=(B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    la = -np.log1p(np.exp(r.normal(-2, 1, size=gs)))
    if spike:
        la[:, ::9] -= 6.0
    return dict(q=r.normal(size=(B, T, H, dk)), k=k, v=r.normal(size=(B, T, H, dv)),
                log_decay=la, erase=1 / (1 + np.exp(-r.normal(size=gs))),
                write=1 / (1 + np.exp(-r.normal(size=gs))),
                S0=r.normal(0, 0.3, size=(B, H, dk, dv)) if s0 else None)


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("chunk", [1, 2, 4, 16, 64])
@pytest.mark.parametrize("gates", ["key", "head"])
@pytest.mark.parametrize("tied", [False, True])
def test_chunk_form_equals_recurrence(chunk, gates, tied):
    c = _case(100 + chunk, gates=gates, spike=True)
    w = None if tied else c["write"]
    o_ref, S_ref = gdn2_forward(c["q"], c["k"], c["v"], c["log_decay"], c["erase"], w, c["S0"],
                                q_scale=0.7)
    o, S = chunk_forward(c["q"], c["k"], c["v"], c["log_decay"], c["erase"], w, c["S0"],
                         chunk=chunk, q_scale=0.7)
    assert _rel(o, o_ref) < 1e-12
    assert _rel(S, S_ref) < 1e-12


def test_chunk_form_zero_state_and_mixed_kinds():
    c = _case(7, T=50, s0=False)
    la_head = c["log_decay"][..., 0]
    o_ref, S_ref = gdn2_forward(c["q"], c["k"], c["v"], la_head, c["erase"], c["write"][..., 0])
    o, S = chunk_forward(c["q"], c["k"], c["v"], la_head, c["erase"], c["write"][..., 0], chunk=16)
    assert _rel(o, o_ref) < 1e-12 and _rel(S, S_ref) < 1e-12
