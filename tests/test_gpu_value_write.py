"""GPU parity of the value-write form (desc->form = GDN2_FORM_VALUE_WRITE).

The gist.science summary's equation, S = (I - k (b .* k)^T) Diag(a) S + k (w .* v)^T
with a write gate per value channel, against the oracle's value-write form on
the same values: the two-pass matrix-core kernels (bf16, d = 128, C = 64),
the general fp32 kernel (any other request, and the bf16 request without a
workspace), and the decode step.  Same tolerances as the key-axis form.
"""
import numpy as np
import pytest

from gated_delta_rule_decay_amd import synth
from oracle.oracle import gdn2_forward
from tests.parity_util import TOL_BF16, TOL_F32, check_every_chain, rel_l2, to_device

pytestmark = pytest.mark.gpu
W = synth.WORKLOADS


def _inputs(w, seed, gates="key"):
    """The workload recipe, with the write gate drawn per value channel
    (``gates="kda"``: the decay per key channel, the erase and write rates
    one per token-head)."""
    inp = synth.make_inputs(w.scaled(gates="head" if gates == "head" else "key", tied=False), seed=seed)
    r = np.random.Generator(np.random.PCG64(seed + 1))
    shape = (w.B, w.T, w.H, w.dv) if gates == "key" else (w.B, w.T, w.H)
    inp["write"] = (1 / (1 + np.exp(-r.standard_normal(shape)))).astype(np.float32)
    if gates == "kda":
        inp["erase"] = np.ascontiguousarray(inp["erase"][..., 0])
    return inp


def _check(w, inp, chunk, ws=True, tol=None, chains=None):
    import torch
    from gated_delta_rule_decay_amd import chunk_fwd

    d = to_device(inp)
    o, S = chunk_fwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"],
                     chunk=chunk, workspace=ws, value_write=True)
    torch.cuda.synchronize()
    o, S = o.cpu().numpy(), S.cpu().numpy()
    if chains is None:
        o_ref, S_ref = gdn2_forward(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"],
                                    inp["write"], inp["S0"], value_write=True)
    else:
        sl = lambda x, b, h: x[b:b + 1, :, h:h + 1]
        refs = [gdn2_forward(sl(inp["q"], b, h), sl(inp["k"], b, h), sl(inp["v"], b, h),
                             sl(inp["log_decay"], b, h), sl(inp["erase"], b, h), sl(inp["write"], b, h),
                             None if inp["S0"] is None else inp["S0"][b:b + 1, h:h + 1], value_write=True)
                for b, h in chains]
        o = np.stack([o[b, :, h] for b, h in chains])
        S = np.stack([S[b, h] for b, h in chains])
        o_ref = np.stack([r[0][0, :, 0] for r in refs])
        S_ref = np.stack([r[1][0, 0] for r in refs])
    tol = tol or (TOL_F32 if w.qkv_dtype == "f32" else TOL_BF16)
    eo, es = rel_l2(o, o_ref), rel_l2(S, S_ref)
    print(f"  rel_l2 o={eo:.3e} S={es:.3e} (tol {tol:.0e})", flush=True)
    assert np.isfinite(o).all() and np.isfinite(S).all()
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("ws", [True, False], ids=["two-pass", "general"])
@pytest.mark.parametrize("gates", ["key", "head", "kda"])
def test_bf16_d128(gates, ws):
    w = W[2].scaled(B=1, T=200, H=2)
    _check(w, _inputs(w, 600, gates), 64, ws=ws)


def test_fp32_general_shapes():
    w = W[2].scaled(B=2, T=37, H=1, dk=48, dv=80, qkv_dtype="f32")
    _check(w, _inputs(w, 610), 16)


def test_segmented_scan_and_exact_chunks():
    # 48 chunks on one chain: three segments.  Then queries scaled by 2^18
    # (exact in bf16) put the factored query operand past the fp16 operand
    # bound in every chunk, so every chunk is flagged and run as the exact
    # fp32 token recurrence, which the error then shows (fp32 level, not fp16
    # level).  Queries of 2^10 with a write gate of ~1000 stay on the fast
    # path (every fp16 value in range) at fp16 accuracy.
    w = W[2].scaled(B=1, T=64 * 48, H=1)
    _check(w, _inputs(w, 620), 64)
    inp = _inputs(w, 621)
    inp["q"] = inp["q"] * 1024.0
    inp["q_bf16"] = (inp["q_bf16"].astype(np.uint32) + (10 << 7)).astype(np.uint16)
    inp["write"] = inp["write"] * 1000.0
    _check(w, inp, 64)
    inp = _inputs(w, 621)
    inp["q"] = inp["q"] * np.float32(2.0 ** 18)
    inp["q_bf16"] = (inp["q_bf16"].astype(np.uint32) + (18 << 7)).astype(np.uint16)
    _check(w, inp, 64, tol=1e-5)


def test_full_size_every_chain():
    import torch
    from gated_delta_rule_decay_amd import chunk_fwd

    w = W[2]
    inp = _inputs(w, 630)
    d = to_device(inp)
    o, S = chunk_fwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"],
                     chunk=64, value_write=True)
    torch.cuda.synchronize()
    o_ref, S_ref = gdn2_forward(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"],
                                inp["S0"], value_write=True)
    check_every_chain("gdn2-bf16 value-write form", [("o", o.cpu().numpy(), o_ref, (1, 3)),
                                                     ("S", S.cpu().numpy(), S_ref, (2, 3))], TOL_BF16)


@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, "bf16"), (48, 80, "f32")])
def test_decode_steps(dk, dv, dtype):
    import torch
    from gated_delta_rule_decay_amd import recurrent_step

    w = W[2].scaled(B=3, T=12, H=2, dk=dk, dv=dv, qkv_dtype=dtype)
    inp = _inputs(w, 640)
    d = to_device(inp)
    st = d["S0"].clone()
    outs = []
    for t in range(w.T):
        g = lambda x: x[:, t].contiguous()
        outs.append(recurrent_step(g(d["q"]), g(d["k"]), g(d["v"]), g(d["log_decay"]), g(d["erase"]),
                                   g(d["write"]), st, value_write=True))
    torch.cuda.synchronize()
    o = torch.stack(outs, 1).cpu().numpy()
    o_ref, S_ref = gdn2_forward(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"],
                                inp["write"], inp["S0"], value_write=True)
    tol = TOL_F32 if dtype == "f32" else 1e-5  # decode is fp32 throughout
    assert rel_l2(o, o_ref) <= tol and rel_l2(st.cpu().numpy(), S_ref) <= tol
