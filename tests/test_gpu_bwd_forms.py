"""GPU parity of the backward for the value-write form and for fused input
preparation (gdn2_chunk_bwd with desc->form, desc->gate_logits,
desc->qk_l2norm), against fp64 autograd of the token recurrence
(oracle/oracle_bwd.py: the value-write recurrence, and the input preparation
-softplus / sigmoid / L2 normalisation in front of it).

The gradients of raw inputs are those of the logits and of unnormalised q, k.
Both paths are covered: the matrix-core kernels (dk = dv = 128) and the
general fp32 kernels (other head sizes).  Same fp32 tolerance as the key-form
backward, 1e-5 relative L2 per gradient tensor.
"""
import numpy as np
import pytest

from gated_delta_rule_decay_amd import synth
from oracle.oracle_bwd import gdn2_backward
from tests.parity_util import rel_l2

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
TOL = 1e-5
NAMES = ("dq", "dk", "dv", "d_log_decay", "d_erase", "d_write", "d_state0")
GATES = {False: ("log_decay", "erase", "write"), True: ("x_decay", "x_erase", "x_write")}


def _dev(x, bits=None):
    import torch
    if bits is not None:
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def _value_gate(inp, name, w, seed, raw):
    """Redraw the write gate (or its logit) with one factor per value channel."""
    r = np.random.Generator(np.random.PCG64(seed))
    shape = (w.B, w.T, w.H, w.dv) if w.gates == "key" else (w.B, w.T, w.H)
    x = r.standard_normal(shape).astype(np.float32)
    if raw:  # bf16 logits: the exact values and their bits
        inp[name], inp[name + "_bf16"] = synth.round_to_bf16(x)
    else:
        inp[name] = (1 / (1 + np.exp(-x))).astype(np.float32)


def _run(w, inp, chunk, seed, vw=False, raw=False, norm=True, chains=None):
    import torch
    from gated_delta_rule_decay_amd import chunk_bwd

    r = np.random.Generator(np.random.PCG64(seed))
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    d_o = r.standard_normal((B, T, H, dv)).astype(np.float32)
    d_st = r.standard_normal((B, H, dk, dv)).astype(np.float32)
    ga, gb, gw = GATES[raw]
    q, k, v = (_dev(inp[n], inp.get(n + "_bf16")) for n in ("q", "k", "v"))
    gates = [_dev(inp[n], inp.get(n + "_bf16") if raw else None) for n in (ga, gb, gw)]
    g = chunk_bwd(q, k, v, *gates, _dev(inp["S0"]), _dev(d_o), _dev(d_st), chunk=chunk,
                  value_write=vw, qk_l2norm=raw and norm)
    torch.cuda.synchronize()
    got = {key: (None if x is None else x.cpu().numpy()) for key, x in g.items()}
    chains = chains or [(b, h) for b in range(B) for h in range(H)]
    sl = lambda x, b, h: None if x is None else x[b:b + 1, :, h:h + 1]
    st = lambda x, b, h: None if x is None else x[b:b + 1, h:h + 1]
    refs = [gdn2_backward(sl(inp["q"], b, h), sl(inp["k"], b, h), sl(inp["v"], b, h), sl(inp[ga], b, h),
                          sl(inp[gb], b, h), sl(inp.get(gw), b, h), st(inp["S0"], b, h), sl(d_o, b, h),
                          st(d_st, b, h), value_write=vw, raw=raw, qk_l2norm=norm)
            for b, h in chains]
    pick = lambda x, b, h, key: x[b:b + 1, h:h + 1] if key == "d_state0" else x[b:b + 1, :, h:h + 1]
    errs = {}
    for key in NAMES:
        if refs[0][key] is None:
            assert got[key] is None
            continue
        gk = np.concatenate([pick(got[key], b, h, key) for b, h in chains])
        rk = np.concatenate([rf[key] for rf in refs])
        assert gk.shape == rk.shape and np.isfinite(gk).all(), key
        errs[key] = rel_l2(gk, rk)
    print("  " + " ".join(f"{kk}={e:.1e}" for kk, e in errs.items()), flush=True)
    for key, e in errs.items():
        assert e <= TOL, (key, e)


@pytest.mark.parametrize("gates", ["key", "head"])
def test_value_write_d128(gates):
    w = W[2].scaled(B=1, T=100, H=2, gates=gates)
    inp = synth.make_inputs(w, seed=800)
    _value_gate(inp, "write", w, 801, raw=False)
    _run(w, inp, 64, seed=802, vw=True)


def test_value_write_segmented():
    # one chain of 3072 tokens: the scans in 3 segments (summaries, combine,
    # rescan) with the value-write form's w .* v in the state terms
    w = W[2].scaled(B=1, T=3072, H=1)
    inp = synth.make_inputs(w, seed=810)
    _value_gate(inp, "write", w, 811, raw=False)
    _run(w, inp, 64, seed=812, vw=True)


@pytest.mark.parametrize("gates", ["key", "head"])
def test_value_write_general_shapes(gates):
    w = W[2].scaled(B=2, T=37, H=1, dk=48, dv=80, qkv_dtype="f32", gates=gates)
    inp = synth.make_inputs(w, seed=810)
    _value_gate(inp, "write", w, 811, raw=False)
    _run(w, inp, 16, seed=812, vw=True)


def test_value_write_head_gate_run_to_run_bitwise():
    # the general path's per-head write gradient of the value-write form is a
    # sum over value channels: taken in a fixed order, two calls agree bit for bit
    import torch
    from gated_delta_rule_decay_amd import chunk_bwd

    w = W[2].scaled(B=2, T=70, H=2, dk=48, dv=80, qkv_dtype="f32", gates="head")
    inp = synth.make_inputs(w, seed=815)
    _value_gate(inp, "write", w, 816, raw=False)
    r = np.random.Generator(np.random.PCG64(817))
    d_o = _dev(r.standard_normal((w.B, w.T, w.H, w.dv)))
    d_st = _dev(r.standard_normal((w.B, w.H, w.dk, w.dv)))
    args = [_dev(inp[n]) for n in ("q", "k", "v", "log_decay", "erase", "write", "S0")]
    runs = []
    for _ in range(3):
        g = chunk_bwd(*args, d_o, d_st, chunk=16, value_write=True)
        torch.cuda.synchronize()
        runs.append({k: v.cpu().numpy() for k, v in g.items() if v is not None})
    for n in runs[0]:
        assert np.array_equal(runs[0][n], runs[1][n]) and np.array_equal(runs[0][n], runs[2][n]), n


@pytest.mark.parametrize("gates,tied", [("key", False), ("head", True)])
def test_raw_inputs_d128(gates, tied):
    w = W[2].scaled(B=1, T=90, H=2, gates=gates, tied=tied)
    _run(w, synth.make_raw_inputs(w, seed=820), 64, seed=821, raw=True)


def test_logits_without_norm_d128():
    # gates as logits, q and k normalised on the host (the workload recipe: the
    # same draws), so the kernels do not normalise them
    w = W[2].scaled(B=1, T=70, H=2)
    inp = synth.make_raw_inputs(w, seed=830)
    nrm = synth.make_inputs(w, seed=830)
    for n in ("q", "k"):
        inp[n], inp[n + "_bf16"] = nrm[n], nrm[n + "_bf16"]
    _run(w, inp, 64, seed=831, raw=True, norm=False)


def test_raw_inputs_general_shapes():
    w = W[2].scaled(B=1, T=45, H=2, dk=32, dv=24, qkv_dtype="f32")
    _run(w, synth.make_raw_inputs(w, seed=840), 16, seed=841, raw=True)


@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, "bf16"), (48, 80, "f32")])
def test_raw_inputs_value_write(dk, dv, dtype):
    w = W[2].scaled(B=1, T=66, H=2, dk=dk, dv=dv, qkv_dtype=dtype)
    inp = synth.make_raw_inputs(w, seed=850)
    _value_gate(inp, "x_write", w, 851, raw=True)
    _run(w, inp, 64 if dk == 128 else 16, seed=852, vw=True, raw=True)


def test_full_size_raw_value_write_sampled_chain():
    # the full GDN-2 workload's shape (B8 H16 T4096): every chain runs, one is checked
    w = W[2]
    inp = synth.make_raw_inputs(w, wid=2)
    _value_gate(inp, "x_write", w, 861, raw=True)
    _run(w, inp, 64, seed=862, vw=True, raw=True, chains=[(5, 9)])
