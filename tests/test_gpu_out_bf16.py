"""GPU: the bf16 output option (desc->o_dtype = GDN2_BF16).

Every kernel computes o in fp32 and rounds it to bf16 (nearest even) only
where it stores it, so on the same inputs a bf16-output call must equal the
fp32-output call rounded by torch (bit for bit), and the final state must not
change at all.  Covered: the two-pass kernels (fast and exact chunks), the
single-pass kernel, the general kernel, packed sequences, and both decode
kernels; one case also bounds the bf16 output against the fp64 oracle.
"""
import numpy as np
import pytest

from gated_delta_rule_decay_amd import synth
from tests.parity_util import TOL_BF16, oracle_chunk, rel_l2, to_device

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _same_rounded(o32, o16):
    import torch
    assert o16.dtype == torch.bfloat16 and o32.dtype == torch.float32
    ref = o32.to(torch.bfloat16)
    assert torch.equal(ref.view(torch.int16), o16.view(torch.int16)), \
        f"{(ref.view(torch.int16) != o16.view(torch.int16)).sum().item()} elements differ"


def _both(fn):
    import torch
    o32, s32 = fn(torch.float32)
    o16, s16 = fn(torch.bfloat16)
    torch.cuda.synchronize()
    _same_rounded(o32, o16)
    if s32 is not None:
        assert torch.equal(s32, s16)
    return o16


def _chunk(inp, chunk=64, **kw):
    from gated_delta_rule_decay_amd import chunk_fwd

    d = to_device(inp)
    return _both(lambda dt: chunk_fwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"],
                                      d["S0"], chunk=chunk, out_dtype=dt, **kw))


@pytest.mark.parametrize("ws", [True, False], ids=["two-pass", "one-pass"])
def test_bf16_workload(ws):
    w = W[2].scaled(B=1, T=200, H=2)
    inp = synth.make_inputs(w, seed=3100)
    o16 = _chunk(inp, workspace=ws)
    o_ref, _ = oracle_chunk(inp)
    e = rel_l2(o16.float().cpu().numpy(), o_ref)
    print(f"  rel_l2 o(bf16)={e:.3e}", flush=True)
    assert e <= TOL_BF16


def test_exact_chunks():
    # |S| beyond the fp16 operand range: the chunks take the exact recurrence,
    # which stores o through its own path
    w = W[2].scaled(B=1, T=150, H=2)
    inp = synth.make_inputs(w, seed=3110)
    inp["S0"] = inp["S0"] * 3.0e5
    _chunk(inp)


def test_general_kernel():
    w = W[2].scaled(B=2, T=45, H=2, dk=48, dv=80, qkv_dtype="f32")
    _chunk(synth.make_inputs(w, seed=3120), chunk=16)


def test_long_sequence_segments():
    # one chain of 4200 tokens: the two-level scan writes o in its last launch
    w = W[3].scaled(B=1, T=4200, H=1)
    _chunk(synth.make_inputs(w, seed=3130))


def test_packed_sequences():
    import torch
    from gated_delta_rule_decay_amd import chunk_fwd_varlen

    w = W[2].scaled(B=1, T=300, H=2)
    lengths = [120, 1, 0, 179]
    inp = synth.make_packed_inputs(w, lengths, seed=3140)
    d = to_device(inp)
    cu = torch.from_numpy(synth.packed_offsets(lengths)).cuda()
    flat = lambda x: None if x is None else x.reshape((-1,) + tuple(x.shape[2:]))
    _both(lambda dt: chunk_fwd_varlen(flat(d["q"]), flat(d["k"]), flat(d["v"]), flat(d["log_decay"]),
                                      flat(d["erase"]), flat(d["write"]), cu, d["S0"], out_dtype=dt))


@pytest.mark.parametrize("dk,dtype", [(128, "bf16"), (48, "f32")])
def test_decode(dk, dtype):
    import torch
    from gated_delta_rule_decay_amd import recurrent_step

    w = W[4].scaled(B=5, H=3, dk=dk, dv=dk, qkv_dtype=dtype)
    st = synth.make_decode_state(w)
    step = to_device(synth.make_decode_step(w, 0))

    def run(dt):
        s = torch.from_numpy(np.ascontiguousarray(st)).cuda()
        o = recurrent_step(step["q"], step["k"], step["v"], step["log_decay"], step["erase"],
                           step["write"], s, out_dtype=dt)
        return o, s

    _both(run)
