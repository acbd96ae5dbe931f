"""GPU check of gdn2_chunk_fwd_static, the forward that allocates nothing:
its output against gdn2_chunk_fwd's (the same request with a workspace), on
two calls in a row, the second with a smaller input.

Where both run the plain scan (enough chains that the workspace form does not
cut sequences into segments) the static form runs the same kernels on the
same values, window by window with the state carried in fp32, so the results
must agree bit for bit; where the workspace form scans in segments the two
differ by rounding only and are held to the bf16 bar (relative L2 <= 2e-3,
and each against the fp64 oracle too).
"""
import numpy as np
import pytest

from gated_delta_rule_decay_amd import synth
from tests.parity_util import TOL_BF16, oracle_chunk, rel_l2, to_device

pytestmark = pytest.mark.gpu
W = synth.WORKLOADS


def _both(w, inp, state0=True, state_out=True):
    import torch
    from gated_delta_rule_decay_amd import chunk_fwd, chunk_fwd_static

    d = to_device(inp)
    s0 = d["S0"] if state0 else None
    args = (d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], s0)
    o_ws, s_ws = chunk_fwd(*args, chunk=w.chunk, workspace=True)
    o = torch.full_like(o_ws, float("nan"))
    st = torch.full_like(s_ws, float("nan")) if state_out else None
    o_st, s_st = chunk_fwd_static(*args, chunk=w.chunk, out=o, state_out=st, return_state=state_out)
    torch.cuda.synchronize()
    return (o_ws.cpu().numpy(), s_ws.cpu().numpy(), o_st.cpu().numpy(),
            None if s_st is None else s_st.cpu().numpy())


def test_static_forward_equals_the_workspace_forward_two_calls():
    # first call: the full GDN-2 workload (128 chains x 64 chunks: 564 MiB of
    # records, so the static form runs 13-chunk windows, the state carried
    # between them); second call smaller (one window)
    w = W[2]
    o_ws, s_ws, o_st, s_st = _both(w, synth.make_inputs(w, wid=2))
    print(f"  full size: o equal {np.array_equal(o_ws, o_st)}, S equal {np.array_equal(s_ws, s_st)}", flush=True)
    assert np.array_equal(o_ws, o_st) and np.array_equal(s_ws, s_st)
    w2 = W[2].scaled(B=2, T=300, H=32)
    o_ws, s_ws, o_st, s_st = _both(w2, synth.make_inputs(w2, seed=1201))
    assert np.array_equal(o_ws, o_st) and np.array_equal(s_ws, s_st)


def test_static_forward_windows_without_state_tensors():
    # no initial state and no final state requested: the windows still carry
    # the state through the scratch
    w = W[2].scaled(B=16, T=2048, H=16)   # 256 chains x 32 chunks: windows of 6
    o_ws, s_ws, o_st, s_st = _both(w, synth.make_inputs(w, seed=1202), state0=False, state_out=False)
    assert s_st is None and np.array_equal(o_ws, o_st)


@pytest.mark.parametrize("gates,tied", [("key", False), ("head", True)])
def test_static_forward_few_chains_long_sequence(gates, tied):
    # two chains of 48 chunks: the workspace form scans them in segments, the
    # static form in one plain scan; both within the bf16 bar of each other
    # and of the oracle
    w = W[2].scaled(B=1, T=64 * 48 - 7, H=2, gates=gates, tied=tied)
    inp = synth.make_inputs(w, seed=1203)
    o_ws, s_ws, o_st, s_st = _both(w, inp)
    o_ref, s_ref = oracle_chunk(inp)
    for x, ref in ((o_st, o_ws), (s_st, s_ws), (o_st, o_ref), (s_st, s_ref)):
        assert np.isfinite(x).all() and rel_l2(x, ref) <= TOL_BF16


def test_static_forward_without_a_two_pass_kernel():
    # fp32 inputs: the general kernel, which uses no scratch at all
    w = W[2].scaled(B=1, T=90, H=2, qkv_dtype="f32", chunk=32)
    inp = synth.make_inputs(w, seed=1204)
    o_ws, s_ws, o_st, s_st = _both(w, inp)
    assert np.array_equal(o_ws, o_st) and np.array_equal(s_ws, s_st)
