"""GPU parity of the fused input preparation (desc->gate_logits, desc->qk_l2norm).

Gates arrive as bf16 logits (log a = -softplus(x), b = w = sigmoid(x) in the
kernels) and q, k unnormalised (divided by their L2 norm in the kernels);
the oracle applies the same preparation in fp64 (oracle.prepare_inputs) to
exactly the same values and runs the recurrence.  Covers the two-pass
matrix-core kernels (including the value-write form, the two-level scan and
the exact path), the general fp32 kernel, and the decode step.
"""
import numpy as np
import pytest

from gated_delta_rule_decay_amd import synth
from oracle.oracle import gdn2_forward_raw
from tests.parity_util import TOL_BF16, TOL_F32, check_every_chain, rel_l2

pytestmark = pytest.mark.gpu
W = synth.WORKLOADS


def _dev(inp, logits=True, norm=True):
    """Device tensors: raw q, k (or the normalised ones), gates as bf16
    logits (or activated fp32)."""
    import torch

    def t(vals, bits):
        if bits is not None:
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
        return None if vals is None else torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float32)).cuda()

    d = {n: t(inp[n], inp.get(n + "_bf16")) for n in ("q", "k", "v")}
    for n in ("x_decay", "x_erase", "x_write"):
        d[n] = t(inp[n], inp.get(n + "_bf16"))
    d["S0"] = None if inp["S0"] is None else torch.from_numpy(inp["S0"]).cuda()
    return d


def _check(w, inp, chunk=64, ws=True, norm=True, value_write=False, tol=None):
    import torch
    from gated_delta_rule_decay_amd import chunk_fwd

    d = _dev(inp)
    o, S = chunk_fwd(d["q"], d["k"], d["v"], d["x_decay"], d["x_erase"], d["x_write"], d["S0"], chunk=chunk,
                     workspace=ws, value_write=value_write, qk_l2norm=norm)
    torch.cuda.synchronize()
    o_ref, S_ref = gdn2_forward_raw(inp["q"], inp["k"], inp["v"], inp["x_decay"], inp["x_erase"],
                                    inp["x_write"], inp["S0"], qk_l2norm=norm, value_write=value_write)
    tol = tol or (TOL_F32 if w.qkv_dtype == "f32" else TOL_BF16)
    eo, es = rel_l2(o.cpu().numpy(), o_ref), rel_l2(S.cpu().numpy(), S_ref)
    print(f"  rel_l2 o={eo:.3e} S={es:.3e} (tol {tol:.0e})", flush=True)
    assert eo <= tol and es <= tol
    return o, S


@pytest.mark.parametrize("ws", [True, False], ids=["two-pass", "general"])
@pytest.mark.parametrize("gates,tied", [("key", False), ("head", True)])
def test_logits_and_norm_bf16_d128(gates, tied, ws):
    w = W[2].scaled(B=1, T=200, H=2, gates=gates, tied=tied)
    _check(w, synth.make_raw_inputs(w, seed=700), ws=ws)


@pytest.mark.parametrize("ws", [True, False], ids=["two-pass", "general"])
def test_kda_gate_logits(ws):
    # KDA's gates as logits: the decay logit per key channel, one erase-rate
    # logit per token-head (tied write)
    w = W[2].scaled(B=1, T=170, H=2, tied=True)
    inp = synth.make_raw_inputs(w, seed=705)
    inp["x_erase"] = np.ascontiguousarray(inp["x_erase"][..., 0])
    inp["x_erase_bf16"] = np.ascontiguousarray(inp["x_erase_bf16"][..., 0])
    _check(w, inp, ws=ws)


def test_full_size_every_chain():
    # the GDN-2 workload's draws as raw inputs (bf16 gate logits, q and k
    # unnormalised), as the bench times them: the two-pass kernels with both
    # preparations fused, every chain against the oracle's fp64 preparation
    # and recurrence
    import torch
    from gated_delta_rule_decay_amd import chunk_fwd

    w = W[2]
    inp = synth.make_raw_inputs(w, wid=2)
    d = _dev(inp)
    o, S = chunk_fwd(d["q"], d["k"], d["v"], d["x_decay"], d["x_erase"], d["x_write"], d["S0"], chunk=w.chunk,
                     qk_l2norm=True)
    torch.cuda.synchronize()
    o_ref, S_ref = gdn2_forward_raw(inp["q"], inp["k"], inp["v"], inp["x_decay"], inp["x_erase"],
                                    inp["x_write"], inp["S0"], qk_l2norm=True)
    check_every_chain(f"{w.name} raw inputs", [("o", o.cpu().numpy(), o_ref, (1, 3)),
                                             ("S", S.cpu().numpy(), S_ref, (2, 3))], TOL_BF16)


def test_logits_without_norm():
    # q, k normalised on the host (the workload recipe), gates as logits
    w = W[2].scaled(B=1, T=150, H=2)
    inp = synth.make_raw_inputs(w, seed=710)
    nrm = synth.make_inputs(w, seed=710)   # same draws, q/k normalised
    for n in ("q", "k"):
        inp[n], inp[n + "_bf16"] = nrm[n], nrm[n + "_bf16"]
    _check(w, inp, norm=False)


def test_fp32_general_shapes():
    w = W[2].scaled(B=2, T=37, H=1, dk=48, dv=80, qkv_dtype="f32")
    _check(w, synth.make_raw_inputs(w, seed=720), chunk=16)


def test_value_write_form():
    w = W[2].scaled(B=1, T=130, H=2)
    inp = synth.make_raw_inputs(w, seed=730)
    _check(w, inp, value_write=True)


def test_segmented_scan_and_exact_chunks():
    # three segments; then a state beyond the fp16 range sends chunks to the
    # exact path, which activates the logits and normalises q, k itself
    w = W[2].scaled(B=1, T=64 * 48, H=1)
    _check(w, synth.make_raw_inputs(w, seed=740))
    inp = synth.make_raw_inputs(w, seed=741)
    inp["S0"] = inp["S0"] * 3.0e5
    _check(w, inp)


def test_scaling_q_k_changes_nothing():
    import torch
    from gated_delta_rule_decay_amd import chunk_fwd

    w = W[2].scaled(B=1, T=100, H=2)
    inp = synth.make_raw_inputs(w, seed=750)
    d = _dev(inp)
    args = lambda q, k: (q, k, d["v"], d["x_decay"], d["x_erase"], d["x_write"], d["S0"])
    o1, S1 = chunk_fwd(*args(d["q"], d["k"]), qk_l2norm=True)
    o2, S2 = chunk_fwd(*args(d["q"] * 4, d["k"] * 0.25), qk_l2norm=True)  # exact in bf16
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, "bf16"), (48, 80, "f32")])
def test_decode_steps(dk, dv, dtype):
    import torch
    from gated_delta_rule_decay_amd import recurrent_step

    w = W[2].scaled(B=3, T=10, H=2, dk=dk, dv=dv, qkv_dtype=dtype)
    inp = synth.make_raw_inputs(w, seed=760)
    d = _dev(inp)
    st = d["S0"].clone()
    outs = []
    for t in range(w.T):
        g = lambda x: x[:, t].contiguous()
        outs.append(recurrent_step(g(d["q"]), g(d["k"]), g(d["v"]), g(d["x_decay"]), g(d["x_erase"]),
                                   g(d["x_write"]), st, qk_l2norm=True))
    torch.cuda.synchronize()
    o = torch.stack(outs, 1).cpu().numpy()
    o_ref, S_ref = gdn2_forward_raw(inp["q"], inp["k"], inp["v"], inp["x_decay"], inp["x_erase"],
                                    inp["x_write"], inp["S0"])
    assert rel_l2(o, o_ref) <= 1e-5 and rel_l2(st.cpu().numpy(), S_ref) <= 1e-5
