"""GPU parity of the chunkwise backward (gdn2_chunk_bwd) against the gradient oracle.

Seeded inputs with the workloads' recipe plus seeded cotangents d_o and
d_state (standard normal); the library's gradients are compared with fp64
autograd of the token recurrence (oracle/oracle_bwd.py) on exactly the same
values, tensor by tensor, by relative L2 error.  The backward computes in
fp32 whatever the q/k/v dtype (bf16 inputs are exact in fp32), so one bound
serves both: the fp32 tolerance of the forward, 1e-5.  The cases measure
1e-7 .. 7e-7 (printed): fp32 rounding of sums of a few hundred terms.
"""
import numpy as np
import pytest

from gated_delta_rule_decay_amd import synth
from oracle.oracle_bwd import gdn2_backward
from tests.parity_util import check_every_chain, rel_l2, to_device

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
TOL = 1e-5
NAMES = ("dq", "dk", "dv", "d_log_decay", "d_erase", "d_write", "d_state0")


def _run(w, inp, chunk, seed, q_scale=1.0, with_dstate=True, chains=None):
    import torch
    from gated_delta_rule_decay_amd import chunk_bwd

    r = np.random.Generator(np.random.PCG64(seed))
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    d_o = r.standard_normal((B, T, H, dv)).astype(np.float32)
    d_st = r.standard_normal((B, H, dk, dv)).astype(np.float32) if with_dstate else None
    d = to_device(inp)
    g = chunk_bwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"],
                  torch.from_numpy(d_o).cuda(), None if d_st is None else torch.from_numpy(d_st).cuda(),
                  chunk=chunk, q_scale=q_scale)
    torch.cuda.synchronize()
    got = {k: (None if v is None else v.cpu().numpy()) for k, v in g.items()}
    if chains is None:
        ref = gdn2_backward(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"],
                            inp["S0"], d_o, d_st, q_scale=q_scale)
        return got, ref
    # independent (batch, head) chains: the oracle on the sampled ones only
    sl = lambda x, b, h: None if x is None else x[b:b + 1, :, h:h + 1]
    st = lambda x, b, h: None if x is None else x[b:b + 1, h:h + 1]
    refs = []
    for b, h in chains:
        refs.append(gdn2_backward(sl(inp["q"], b, h), sl(inp["k"], b, h), sl(inp["v"], b, h),
                                  sl(inp["log_decay"], b, h), sl(inp["erase"], b, h),
                                  sl(inp["write"], b, h), st(inp["S0"], b, h), sl(d_o, b, h),
                                  st(d_st, b, h), q_scale=q_scale))
    pick = lambda x, b, h, key: x[b:b + 1, h:h + 1] if key == "d_state0" else x[b:b + 1, :, h:h + 1]
    got_s, ref_s = {}, {}
    for key in NAMES:
        if got[key] is None:
            got_s[key] = ref_s[key] = None
            continue
        got_s[key] = np.concatenate([pick(got[key], b, h, key) for b, h in chains])
        ref_s[key] = np.concatenate([rf[key] for rf in refs])
    return got_s, ref_s


def _compare(got, ref, tol=TOL):
    errs = {}
    for key in NAMES:
        if ref.get(key) is None:
            assert got.get(key) is None
            continue
        assert got[key].shape == ref[key].shape, key
        assert np.isfinite(got[key]).all(), key
        errs[key] = rel_l2(got[key], ref[key])
    print("  " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    for key, e in errs.items():
        assert e <= tol, (key, e)


def test_tiny_fp32_workload():
    w = W[0]
    _compare(*_run(w, synth.make_inputs(w, wid=0), w.chunk, seed=200))


@pytest.mark.parametrize("wid,B,T,H,chunk", [(2, 1, 100, 2, 64), (2, 2, 37, 1, 16), (1, 1, 70, 2, 64),
                                             (2, 1, 1, 1, 64)])
def test_reduced_bf16_workloads(wid, B, T, H, chunk):
    w = W[wid].scaled(B=B, T=T, H=H)
    _compare(*_run(w, synth.make_inputs(w, seed=300 + T), chunk, seed=301 + T))


@pytest.mark.parametrize("dtype,dk,dv,T,gates,tied", [("f32", 48, 80, 37, "head", False),
                                                       ("f32", 32, 32, 50, "key", True),
                                                       ("bf16", 64, 64, 45, "head", True),
                                                       ("f32", 16, 24, 33, "key", False)])
def test_shapes_and_gate_kinds(dtype, dk, dv, T, gates, tied):
    w = W[2].scaled(B=1, T=T, H=2, dk=dk, dv=dv, qkv_dtype=dtype, gates=gates, tied=tied)
    _compare(*_run(w, synth.make_inputs(w, seed=400 + dk), 32, seed=401 + dk))


def test_mixed_gate_kinds_and_q_scale():
    # per-head decay, per-channel erase and write, no final-state cotangent
    w = W[2].scaled(B=1, T=60, H=2)
    inp = synth.make_inputs(w, seed=500)
    inp["log_decay"] = np.ascontiguousarray(inp["log_decay"][..., 0])
    _compare(*_run(w, inp, 64, seed=501, q_scale=0.5, with_dstate=False))


def test_zero_initial_state_and_strong_decay():
    w = W[2].scaled(B=1, T=90, H=1)
    inp = synth.make_inputs(w, seed=510)
    inp["S0"] = None
    inp["log_decay"][:, 20:40] = -4.0
    _compare(*_run(w, inp, 64, seed=511))


def test_steep_decay_chunks():
    # channels decaying by 12 nats a token over two 16-token chunks (180 nats
    # within a chunk, where factors around the chunk's middle would pass
    # e^88 and overflow): those chunks' Gram gradients take the direct path
    # (pairwise decays formed one by one), the others the factored
    # matrix-core path
    w = W[2].scaled(B=1, T=80, H=2)
    inp = synth.make_inputs(w, seed=540)
    inp["log_decay"][:, 16:48, :, :8] = -12.0
    _compare(*_run(w, inp, 64, seed=541))


def test_empty_sequence_passes_the_state_gradient():
    import torch
    from gated_delta_rule_decay_amd import chunk_bwd

    w = W[2].scaled(B=2, T=0, H=2)
    inp = synth.make_inputs(w, seed=520)
    d = to_device(inp)
    d_st = torch.randn(2, 2, 128, 128, device="cuda")
    g = chunk_bwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"],
                  torch.zeros(2, 0, 2, 128, device="cuda"), d_st)
    torch.cuda.synchronize()
    assert torch.equal(g["d_state0"], d_st)


def _bwd_full(w, inp, d_o, d_st):
    import torch
    from gated_delta_rule_decay_amd import chunk_bwd

    d = to_device(inp)
    g = chunk_bwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"],
                  torch.from_numpy(d_o).cuda(), torch.from_numpy(d_st).cuda(), chunk=w.chunk)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy()) for k, v in g.items()}


def test_full_size_every_chain():
    # the full GDN-2 workload (B8 H16 T4096, d128), every one of its 128
    # chains against the hand-written fp64 reverse pass of the C oracle
    # (pinned to finite differences and to autograd), per chain; and the
    # same call again, bit for bit
    from oracle.oracle import gdn2_backward_c

    w = W[2]
    inp = synth.make_inputs(w, wid=2)
    r = np.random.Generator(np.random.PCG64(530))
    d_o = r.standard_normal((w.B, w.T, w.H, w.dv)).astype(np.float32)
    d_st = r.standard_normal((w.B, w.H, w.dk, w.dv)).astype(np.float32)
    got = _bwd_full(w, inp, d_o, d_st)
    ref = gdn2_backward_c(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"],
                          inp["S0"], d_o, d_st)
    tok = (1, 3)   # [B,T,H,d]: a chain is (b, h)
    check_every_chain("gdn2-bf16 backward", [(n, got[n], ref[n], (2, 3) if n == "d_state0" else tok)
                                             for n in NAMES], TOL)
    again = _bwd_full(w, inp, d_o, d_st)
    for n in NAMES:
        assert np.array_equal(got[n], again[n]), f"{n} differs between two identical calls"


def test_full_size_gated_deltanet_every_chain():
    # the Gated DeltaNet workload (B4 H16 T4096: one decay and one tied rate
    # per token-head, zero initial state) through the matrix-core backward,
    # every one of its 64 chains against the C oracle's reverse pass
    from oracle.oracle import gdn2_backward_c

    w = W[1]
    inp = synth.make_inputs(w, wid=1)
    r = np.random.Generator(np.random.PCG64(535))
    d_o = r.standard_normal((w.B, w.T, w.H, w.dv)).astype(np.float32)
    d_st = r.standard_normal((w.B, w.H, w.dk, w.dv)).astype(np.float32)
    got = _bwd_full(w, inp, d_o, d_st)
    ref = gdn2_backward_c(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"],
                          inp["S0"], d_o, d_st)
    tok = (1, 3)
    head = (1,)  # per-head gates [B,T,H]: a chain is (b, h), its tokens on axis 1
    axes = {"d_state0": (2, 3), "d_log_decay": head, "d_erase": head}
    check_every_chain("gdn-scalar backward", [(n, got[n], ref[n], axes.get(n, tok))
                                              for n in NAMES if ref[n] is not None], TOL)


@pytest.mark.parametrize("T", [2048, 4001, 4096])
def test_segmented_scans(T):
    # two chains over long sequences: the scans run as segment summaries, the
    # combine and a rescan (2, 3 and 4 segments of 64 to 85 chunks; T = 4001
    # ends in a one-token chunk); every chain against the C reverse pass
    from oracle.oracle import gdn2_backward_c

    w = W[2].scaled(B=1, T=T, H=2)
    inp = synth.make_inputs(w, seed=620 + T)
    r = np.random.Generator(np.random.PCG64(621 + T))
    d_o = r.standard_normal((w.B, w.T, w.H, w.dv)).astype(np.float32)
    d_st = r.standard_normal((w.B, w.H, w.dk, w.dv)).astype(np.float32)
    got = _bwd_full(w, inp, d_o, d_st)
    ref = gdn2_backward_c(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"],
                          inp["S0"], d_o, d_st)
    check_every_chain(f"segmented backward T={T}", [(n, got[n], ref[n], (2, 3) if n == "d_state0" else (1, 3))
                                                    for n in NAMES], TOL)


def test_full_size_long_context_every_chain():
    # the long-context workload (B1 H16 T65536, decay spikes): 16 chains, so
    # the scans run in 8 segments of 512 chunks; every chain against the C
    # reverse pass
    from oracle.oracle import gdn2_backward_c

    w = W[3]
    inp = synth.make_inputs(w, wid=3)
    r = np.random.Generator(np.random.PCG64(640))
    d_o = r.standard_normal((w.B, w.T, w.H, w.dv)).astype(np.float32)
    d_st = r.standard_normal((w.B, w.H, w.dk, w.dv)).astype(np.float32)
    got = _bwd_full(w, inp, d_o, d_st)
    ref = gdn2_backward_c(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"],
                          inp["S0"], d_o, d_st)
    check_every_chain("long-context backward", [(n, got[n], ref[n], (2, 3) if n == "d_state0" else (1, 3))
                                                for n in NAMES], TOL)


def test_segmented_scans_zero_ends_head_gates():
    # 3 segments with no initial state and no final-state cotangent (the
    # summaries and the rescan then start from zero at both ends), one decay
    # per token-head and a tied per-channel rate
    import torch
    from gated_delta_rule_decay_amd import chunk_bwd
    from oracle.oracle import gdn2_backward_c

    w = W[2].scaled(B=1, T=3072, H=2, tied=True)
    inp = synth.make_inputs(w, seed=650)
    inp["S0"] = None
    inp["log_decay"] = np.ascontiguousarray(inp["log_decay"][..., 0])
    r = np.random.Generator(np.random.PCG64(651))
    d_o = r.standard_normal((w.B, w.T, w.H, w.dv)).astype(np.float32)
    d = to_device(inp)
    g = chunk_bwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], None, None,
                  torch.from_numpy(d_o).cuda(), None, chunk=w.chunk)
    torch.cuda.synchronize()
    got = {k: (None if v is None else v.cpu().numpy()) for k, v in g.items()}
    ref = gdn2_backward_c(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], None, None, d_o, None)
    axes = {"d_state0": (2, 3), "d_log_decay": (1,)}
    check_every_chain("segmented backward, zero ends", [(n, got[n], ref[n], axes.get(n, (1, 3)))
                                                        for n in NAMES if ref[n] is not None], TOL)
