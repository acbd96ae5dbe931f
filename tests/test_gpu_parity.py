"""GPU parity: the HIP library against the fp64 oracle, element by element.

Every case draws seeded inputs with the workloads' recipe, runs the library
through its C ABI (via the binding) on the GPU, runs the oracle on exactly the
same values on the CPU, and bounds the relative L2 error of o and of the
final state: 1e-5 for fp32 q/k/v, 2e-3 for bf16 q/k/v.  Small cases span
several chunks and a ragged last chunk; full-size cases run the launch the
bench times and check sampled (batch, head) chains, which are independent.
"""
import numpy as np
import pytest

from gated_delta_rule_decay_amd import synth
from tests.parity_util import (MAX_ELEM_FACTOR, TOL_BF16, TOL_F32, check_every_chain, gpu_chunk,
                               oracle_chunk, rel_l2, to_device)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _tol(w):
    return TOL_F32 if w.qkv_dtype == "f32" else TOL_BF16


# The bf16 / dk = dv = 128 / C = 64 requests have two kernels: the two-pass
# form (with a workspace, the default) and the single-pass one (none).
PATHS = [pytest.param(True, id="two-pass"), pytest.param(False, id="one-pass")]


def _check(w, inp, chunk, q_scale=1.0, ws=True):
    o, S = gpu_chunk(inp, chunk, q_scale=q_scale, workspace=ws)
    o_ref, S_ref = oracle_chunk(inp, q_scale=q_scale)
    eo, es = rel_l2(o, o_ref), rel_l2(S, S_ref)
    print(f"  rel_l2 o={eo:.3e} S={es:.3e} (tol {_tol(w):.0e})", flush=True)
    assert np.isfinite(o).all() and np.isfinite(S).all()
    assert eo <= _tol(w) and es <= _tol(w)
    return o, S


def test_tiny_fp32_workload():
    w = W[0]
    _check(w, synth.make_inputs(w, wid=0), w.chunk)


@pytest.mark.parametrize("ws", PATHS)
@pytest.mark.parametrize("wid,B,T,H", [(1, 1, 200, 2), (2, 1, 200, 2), (2, 2, 131, 1),
                                       (3, 1, 4200, 1)])
def test_reduced_bf16_workloads(wid, B, T, H, ws):
    w = W[wid].scaled(B=B, T=T, H=H)
    _check(w, synth.make_inputs(w, seed=1000 + wid * 7 + T), w.chunk, ws=ws)


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_fp32_full_width(chunk):
    w = W[2].scaled(B=1, T=150, H=2, qkv_dtype="f32")
    _check(w, synth.make_inputs(w, seed=77 + chunk), chunk)


@pytest.mark.parametrize("dtype,dk,dv,T", [("f32", 48, 80, 37), ("bf16", 64, 64, 100),
                                           ("f32", 1, 3, 20), ("bf16", 128, 32, 70)])
def test_odd_shapes(dtype, dk, dv, T):
    w = W[2].scaled(B=2, T=T, H=1, dk=dk, dv=dv, qkv_dtype=dtype, chunk=32)
    _check(w, synth.make_inputs(w, seed=dk * 1000 + dv + T), 32)


@pytest.mark.parametrize("ws", PATHS)
@pytest.mark.parametrize("gates,tied", [("head", False), ("key", True), ("head", True)])
def test_gate_kinds(gates, tied, ws):
    w = W[2].scaled(B=1, T=160, H=2, gates=gates, tied=tied)
    _check(w, synth.make_inputs(w, seed=5 + tied), 64, ws=ws)


def _kda_gates(inp, tied):
    # KDA's gates: the per-channel decay kept, one erase (and write) rate per
    # token-head (the first channel's draw)
    inp["erase"] = np.ascontiguousarray(inp["erase"][..., 0])
    inp["write"] = None if tied else np.ascontiguousarray(inp["write"][..., 0])
    return inp


@pytest.mark.parametrize("ws", PATHS)
@pytest.mark.parametrize("tied", [True, False])
def test_kda_gates(tied, ws):
    w = W[2].scaled(B=2, T=230, H=2)
    _check(w, _kda_gates(synth.make_inputs(w, seed=61 + tied), tied), 64, ws=ws)


def test_kda_gates_exact_chunks():
    # a KDA chunk flagged for the exact recurrence (state beyond fp16 range)
    w = W[2].scaled(B=1, T=150, H=2)
    inp = _kda_gates(synth.make_inputs(w, seed=63), True)
    inp["S0"] = inp["S0"] * 3.0e5
    _check(w, inp, 64, ws=True)


@pytest.mark.parametrize("ws", PATHS)
def test_q_scale_and_zero_state(ws):
    w = W[2].scaled(B=1, T=96, H=2, s0_std=0.0)
    _check(w, synth.make_inputs(w, seed=9), 64, q_scale=0.125, ws=ws)


@pytest.mark.parametrize("ws", PATHS)
def test_edge_lengths(ws):
    import torch
    from gated_delta_rule_decay_amd import chunk_fwd

    for T in (1, 63, 64, 65):
        w = W[2].scaled(B=1, T=T, H=1)
        _check(w, synth.make_inputs(w, seed=T), 64, ws=ws)
    # T == 0: the final state is the initial state, o untouched
    w = W[2].scaled(B=1, T=0, H=2)
    d = to_device(synth.make_inputs(w, seed=3))
    o, S = chunk_fwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"])
    torch.cuda.synchronize()
    assert torch.equal(S, d["S0"]) and o.numel() == 0


def test_in_place_state_and_resume():
    import torch
    from gated_delta_rule_decay_amd import chunk_fwd

    w = W[2].scaled(B=1, T=256, H=2)
    inp = synth.make_inputs(w, seed=11)
    d = to_device(inp)
    o_full, S_full = chunk_fwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"],
                               d["S0"])
    # two calls, the second resuming in place from the first's final state
    st = d["S0"].clone()
    sl = lambda x, a, b: None if x is None else x[:, a:b].contiguous()
    o1, _ = chunk_fwd(*(sl(d[n], 0, 128) for n in ("q", "k", "v", "log_decay", "erase", "write")),
                      st, state_out=st)
    o2, _ = chunk_fwd(*(sl(d[n], 128, 256) for n in ("q", "k", "v", "log_decay", "erase", "write")),
                      st, state_out=st)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_chunk(inp)
    assert rel_l2(torch.cat([o1, o2], 1).cpu().numpy(), o_ref) <= TOL_BF16
    assert rel_l2(st.cpu().numpy(), S_ref) <= TOL_BF16
    assert rel_l2(S_full.cpu().numpy(), S_ref) <= TOL_BF16


@pytest.mark.parametrize("ws", PATHS)
def test_run_to_run_bitwise(ws):
    w = W[2].scaled(B=2, T=300, H=2)
    inp = synth.make_inputs(w, seed=12)
    o1, S1 = gpu_chunk(inp, 64, workspace=ws)
    o2, S2 = gpu_chunk(inp, 64, workspace=ws)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def _decode_run(w, steps, seed, sample_heads=None):
    """Run `steps` decode steps on the GPU; returns o per step and the final
    state, plus the inputs of the sampled heads stacked over time."""
    import torch
    from gated_delta_rule_decay_amd import recurrent_step

    import concurrent.futures as cf

    S0 = synth.make_decode_state(w, seed=seed)
    state = torch.from_numpy(S0).cuda()
    outs, keep = [], {n: [] for n in ("q", "k", "v", "log_decay", "erase", "write")}
    pool = cf.ThreadPoolExecutor(max_workers=8)
    batch = 64
    pending = [pool.submit(synth.make_decode_step, w, t, seed) for t in range(min(batch, steps))]
    for t in range(steps):
        inp = pending[t % batch].result()
        if t + batch < steps:
            pending[t % batch] = pool.submit(synth.make_decode_step, w, t + batch, seed)
        d = to_device(inp)
        o = recurrent_step(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], state)
        sel = (slice(None),) if sample_heads is None else (sample_heads[:, 0], sample_heads[:, 1])
        outs.append(o.cpu().numpy()[sel])
        for n in keep:
            if inp[n] is not None:
                keep[n].append(inp[n][sel])
    pool.shutdown()
    torch.cuda.synchronize()
    Sg = state.cpu().numpy()
    if sample_heads is not None:
        Sg = Sg[sample_heads[:, 0], sample_heads[:, 1]]
        S0 = S0[sample_heads[:, 0], sample_heads[:, 1]]
    return np.stack(outs, 1), Sg, S0, {n: (np.stack(v, 1) if v else None) for n, v in keep.items()}


def _decode_oracle(S0, seq):
    """Oracle over the decode sequence: each sampled head is its own chain."""
    from oracle.oracle import gdn2_forward

    add_h = lambda x: None if x is None else x[:, :, None]
    # seq arrays are [n, steps, ...] -> [B=n, T=steps, H=1, ...]
    if S0.ndim == 3:
        S0 = S0[:, None]
    o, S = gdn2_forward(add_h(seq["q"]), add_h(seq["k"]), add_h(seq["v"]), add_h(seq["log_decay"]),
                        add_h(seq["erase"]), add_h(seq["write"]), S0)
    return o[:, :, 0], S[:, 0]


@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, "bf16"), (128, 128, "f32"), (40, 24, "f32")])
def test_decode_small(dk, dv, dtype):
    w = W[4].scaled(B=3, H=2, dk=dk, dv=dv, qkv_dtype=dtype)
    o, S, S0, seq = _decode_run(w, 9, seed=dk + dv)
    n = w.B * w.H
    flat = lambda x: None if x is None else x.reshape((n,) + x.shape[2:])
    # reorder [N, steps, H, ...] -> [N*H, steps, ...]: every head is a chain
    seqf = {k_: None if v_ is None else np.moveaxis(v_, 2, 1).reshape((n, 9) + v_.shape[3:])
            for k_, v_ in seq.items()}
    o_ref, S_ref = _decode_oracle(flat(S0), seqf)
    o_g = np.moveaxis(o, 2, 1).reshape((n, 9, dv))
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert rel_l2(o_g, o_ref) <= tol
    assert rel_l2(flat(S), S_ref) <= tol


def test_decode_steps_equal_chunked_forward():
    import torch
    from gated_delta_rule_decay_amd import chunk_fwd, recurrent_step

    w = W[2].scaled(B=2, T=70, H=2)
    inp = synth.make_inputs(w, seed=21)
    d = to_device(inp)
    o_c, S_c = chunk_fwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"])
    st = d["S0"].clone()
    outs = []
    for t in range(w.T):
        g = lambda x: None if x is None else x[:, t].contiguous()
        outs.append(recurrent_step(g(d["q"]), g(d["k"]), g(d["v"]), g(d["log_decay"]),
                                   g(d["erase"]), g(d["write"]), st))
    torch.cuda.synchronize()
    o_d = torch.stack(outs, 1)
    assert rel_l2(o_d.cpu().numpy(), o_c.cpu().numpy()) <= TOL_BF16
    assert rel_l2(st.cpu().numpy(), S_c.cpu().numpy()) <= TOL_BF16


# ---- full sizes: the exact launches the bench times, every chain -----------

@pytest.mark.parametrize("wid", [1, 2, 3])
def test_full_size_every_chain(wid):
    # every (batch, head) chain of the Gated DeltaNet, GDN-2 and long-context
    # workloads against the oracle, per chain (and the largest element error
    # per chain), on both kernels of the bf16 path: the two-pass form the
    # bench times and the single-pass one
    import torch
    from gated_delta_rule_decay_amd import chunk_fwd

    w = W[wid]
    inp = synth.make_inputs(w, wid=wid)
    o_ref, S_ref = oracle_chunk(inp)
    d = to_device(inp)
    for ws in (True, False):
        o, S = chunk_fwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"],
                         chunk=w.chunk, workspace=ws)
        torch.cuda.synchronize()
        label = f"{w.name} {'two-pass' if ws else 'one-pass'}"
        check_every_chain(label, [("o", o.cpu().numpy(), o_ref, (1, 3)),
                                  ("S", S.cpu().numpy(), S_ref, (2, 3))], TOL_BF16)
        del o, S


def test_full_size_kda_every_chain():
    # KDA's gates on the GDN-2 workload's shape, as the bench times them: the
    # per-channel decay kept, one tied rate per token-head (the first
    # channel's erase draw), the two-pass kernels; every chain against the
    # oracle
    import torch
    from gated_delta_rule_decay_amd import chunk_fwd

    w = W[2]
    inp = synth.make_inputs(w, wid=2)
    inp["erase"] = np.ascontiguousarray(inp["erase"][..., 0])
    inp["write"] = None
    o_ref, S_ref = oracle_chunk(inp)
    d = to_device(inp)
    o, S = chunk_fwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], None, d["S0"], chunk=w.chunk)
    torch.cuda.synchronize()
    check_every_chain(f"{w.name} KDA gates", [("o", o.cpu().numpy(), o_ref, (1, 3)),
                                            ("S", S.cpu().numpy(), S_ref, (2, 3))], TOL_BF16)


def test_full_size_decode_every_head():
    # the decode workload as written: 256 sequences x 16 heads, the fp32 state
    # carried in place across 1024 consecutive steps; every head is checked
    # against the oracle run over the same steps (in blocks of 64 steps,
    # carrying its fp64 state), per head
    import concurrent.futures as cf

    import torch
    from gated_delta_rule_decay_amd import recurrent_step
    from oracle.oracle import gdn2_forward

    w = W[4]
    N, H, dk, dv, steps = w.B, w.H, w.dk, w.dv, w.decode_steps
    n = N * H
    S0 = synth.make_decode_state(w)
    state = torch.from_numpy(S0).cuda()
    ref_state = S0.reshape(n, 1, dk, dv).astype(np.float64)
    o_out = torch.empty((N, H, dv), dtype=torch.float32, device="cuda")
    num = np.zeros(n)
    den = np.zeros(n)
    big = np.zeros(n)
    blk = 64
    pool = cf.ThreadPoolExecutor(max_workers=8)
    futs = {t: pool.submit(synth.make_decode_step, w, t) for t in range(min(2 * blk, steps))}
    for t0 in range(0, steps, blk):
        t1 = min(steps, t0 + blk)
        got, seq = [], []
        for t in range(t0, t1):
            inp = futs.pop(t).result()
            if t + 2 * blk < steps:
                futs[t + 2 * blk] = pool.submit(synth.make_decode_step, w, t + 2 * blk)
            dd = to_device(inp)
            recurrent_step(dd["q"], dd["k"], dd["v"], dd["log_decay"], dd["erase"], dd["write"], state,
                           out=o_out)
            got.append(o_out.cpu().numpy().reshape(n, dv))
            seq.append(inp)
        # [n, steps, 1, ...]: every head is its own chain for the oracle
        stack = lambda name: (None if seq[0][name] is None else
                              np.stack([x[name].reshape((n,) + x[name].shape[2:]) for x in seq], 1)[:, :, None])
        o_ref, ref_state = gdn2_forward(stack("q"), stack("k"), stack("v"), stack("log_decay"),
                                        stack("erase"), stack("write"), ref_state)
        diff = np.stack(got, 1) - o_ref[:, :, 0]
        num += (diff * diff).sum((1, 2))
        den += (o_ref[:, :, 0] ** 2).sum((1, 2))
        big = np.maximum(big, np.abs(diff).max((1, 2)))
    pool.shutdown()
    torch.cuda.synchronize()
    rel_o = np.sqrt(num / den)
    big_o = big / np.sqrt(den / (steps * dv))
    print(f"  decode {steps} steps, {n} heads: o rel_l2 overall {np.sqrt(num.sum() / den.sum()):.3e}, worst head "
          f"{int(np.argmax(rel_o))} {rel_o.max():.3e}, largest element error {big_o.max():.3e} x head RMS",
          flush=True)
    assert np.isfinite(rel_o).all()
    assert rel_o.max() <= TOL_BF16 and big_o.max() <= MAX_ELEM_FACTOR * TOL_BF16
    check_every_chain("decode final state", [("S", state.cpu().numpy().reshape(n, dk, dv),
                                              ref_state[:, 0], (1, 2))], TOL_BF16)


# ---- degenerate gates: the fast path's exact fallback and the limits -------

def _bf16_case(seed, T=200, H=2, B=1, tied=False, gates="key"):
    w = W[2].scaled(B=B, T=T, H=H, tied=tied, gates=gates)
    return w, synth.make_inputs(w, seed=seed)


@pytest.mark.parametrize("ws", PATHS)
def test_near_zero_decay_spikes(ws):
    # a -> 0 on a few tokens and channels: exp(-1000) is 0, the old state is gone there
    w, inp = _bf16_case(31)
    inp["log_decay"][:, 70:73, :, :40] = -1000.0
    inp["log_decay"][:, 130, :, :] = -1000.0
    _check(w, inp, 64, ws=ws)


@pytest.mark.parametrize("ws", PATHS)
def test_strong_uniform_decay(ws):
    # every token decays every channel by e^-3: factors leave fp16 range inside a block
    w, inp = _bf16_case(32)
    inp["log_decay"][:, 64:128] = -3.0
    _check(w, inp, 64, ws=ws)
    w, inp = _bf16_case(33, tied=True, gates="head")
    inp["log_decay"][:] = -2.5
    _check(w, inp, 64, ws=ws)


@pytest.mark.parametrize("ws", PATHS)
def test_no_decay_is_delta_rule(ws):
    w, inp = _bf16_case(34)
    inp["log_decay"][:] = 0.0
    _check(w, inp, 64, ws=ws)


@pytest.mark.parametrize("ws", PATHS)
def test_hold_keeps_state(ws):
    # a = 1 and b = w = 0: the state is held (exactly, since every write is zero)
    import torch
    from gated_delta_rule_decay_amd import chunk_fwd

    w, inp = _bf16_case(35)
    inp["log_decay"][:] = 0.0
    inp["erase"][:] = 0.0
    inp["write"][:] = 0.0
    d = to_device(inp)
    o, S = chunk_fwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"],
                     workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(S, d["S0"])
    _check(w, inp, 64, ws=ws)


# ---- the two-pass form's own cases ---------------------------------------

def test_workspace_reused_across_sizes():
    # one caller-owned workspace, stale records from a larger call first
    import torch
    from gated_delta_rule_decay_amd import chunk_fwd_workspace
    from gated_delta_rule_decay_amd.binding import make_desc

    need = chunk_fwd_workspace(make_desc(2, 300, 2, 128, 128))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for B, T, H, seed in ((2, 300, 2, 41), (1, 70, 2, 42), (1, 1, 1, 43)):
        w = W[2].scaled(B=B, T=T, H=H)
        _check(w, synth.make_inputs(w, seed=seed), 64, ws=ws)
    with pytest.raises(Exception):
        _check(W[2].scaled(B=2, T=400, H=2), synth.make_inputs(W[2].scaled(B=2, T=400, H=2), seed=44),
               64, ws=ws)


@pytest.mark.parametrize("ws", PATHS)
def test_large_state_runs_exactly(ws):
    # |S| beyond the fp16 operand range: those chunks take the exact recurrence
    w, inp = _bf16_case(45, T=200)
    inp["S0"] = inp["S0"] * 3.0e5
    _check(w, inp, 64, ws=ws)


@pytest.mark.parametrize("ws", PATHS)
def test_large_grams_run_exactly(ws):
    # queries scaled by 2^10 (exact in bf16) and a write gate of ~1000: every
    # operand stays in fp16 range but the query Grams do not, so the chunks
    # are flagged and recomputed exactly
    w, inp = _bf16_case(46, T=150)
    inp["q"] = inp["q"] * 1024.0
    inp["q_bf16"] = (inp["q_bf16"].astype(np.uint32) + (10 << 7)).astype(np.uint16)
    inp["write"] = inp["write"] * 1000.0
    _check(w, inp, 64, ws=ws)


@pytest.mark.parametrize("ws", PATHS)
def test_large_query_key_gram_tied(ws):
    # tied gates (the slim two-pass record keeps R itself, not products of
    # it): queries equal to the keys times 2^15 (exact in bf16) and an erase
    # gate of 1 put every diagonal entry of R = (q e^T) at 2^15, past the fp16
    # result bound, while a weak decay (log a = -1e-3) keeps every factored
    # operand within the fp16 operand bound (largest query entry about 1.2e4).
    # Each chunk must be flagged by the Gram's own range check and run as the
    # exact fp32 recurrence: finite results at fp32 accuracy, on both paths.
    w, inp = _bf16_case(48, T=150, tied=True)
    inp["q_bf16"] = _shift_exponent(inp["k_bf16"], 15)
    inp["q"] = inp["k"] * np.float32(2.0 ** 15)
    inp["erase"] = np.ones_like(inp["erase"])
    inp["log_decay"] = np.full_like(inp["log_decay"], -1e-3)
    assert np.abs(inp["q"]).max() < 16384 * 0.99
    o, S = gpu_chunk(inp, 64, workspace=ws)
    o_ref, S_ref = oracle_chunk(inp)
    eo, es = rel_l2(o, o_ref), rel_l2(S, S_ref)
    print(f"  rel_l2 o={eo:.3e} S={es:.3e} (exact path, tol 1e-05)", flush=True)
    assert np.isfinite(o).all() and np.isfinite(S).all()
    assert eo <= 1e-5 and es <= 1e-5


def _shift_exponent(bits, log2):
    """bf16 bits times 2^log2 (exact: the exponent field moves; zeros stay)."""
    b = bits.astype(np.int32)
    return np.where((b & 0x7fff) != 0, b + (log2 << 7), b).astype(np.uint16)


def _scale_bf16(inp, name, log2):
    """Multiply a bf16 input by 2^log2 (exact: the exponent field moves)."""
    bits = inp[name + "_bf16"].astype(np.int32)
    nz = (bits & 0x7fff) != 0
    inp[name + "_bf16"] = np.where(nz, bits + (log2 << 7), bits).astype(np.uint16)
    inp[name] = inp[name] * np.float32(2.0 ** log2)


@pytest.mark.parametrize("ws", PATHS)
def test_header_bound_values_and_state(ws):
    # the bf16 path's stated range: |v| < 2^15 and a state below 2^15.  The
    # products X = Kbar S + Bm V and M of such inputs leave fp16 range; the
    # chunks that do are detected and run exactly, on both paths
    w, inp = _bf16_case(47, T=230)
    _scale_bf16(inp, "v", 12)                        # |v| up to ~2e4
    inp["S0"] = np.clip(inp["S0"] * 2.0e5, -3.2e4, 3.2e4).astype(np.float32)
    assert np.abs(inp["v"]).max() < 2 ** 15
    o, S = _check(w, inp, 64, ws=ws)
    assert np.abs(S).max() < 2 ** 15


@pytest.mark.parametrize("tied", [False, True])
def test_values_past_fp16_run_exactly(tied):
    # values past fp16's range on three tokens of the second chunk (beyond the
    # stated bound |v| < 2^15): untied, the two-pass scan stages the values
    # itself and marks such a chunk for the exact recurrence; tied, the prep
    # pass's D leaves the fp16 range.  Either way the results stay finite and
    # within the bf16 bar (the state then exceeds the fp16 bound, so the later
    # chunks run exactly too)
    w, inp = _bf16_case(49, T=200, tied=tied)
    bits = inp["v_bf16"].astype(np.int32)
    sub = bits[:, 70:73]
    bits[:, 70:73] = np.where((sub & 0x7fff) != 0, sub + (17 << 7), sub)
    inp["v_bf16"] = bits.astype(np.uint16)
    inp["v"][:, 70:73] *= np.float32(2.0 ** 17)
    assert np.abs(inp["v"]).max() > 65504
    _check(w, inp, 64, ws=True)


# ---- the two-level scan: long sequences on few chains ----------------------
# Few (batch, head) chains with many chunks are cut into segments (see
# tests/test_abi.py::segments): 33 chunks -> 2 segments, 48 -> 3, 100 -> 6,
# 64 on two chains -> 4.

@pytest.mark.parametrize("B,H,T,tied,gates", [
    (1, 1, 64 * 33 - 5, False, "key"),
    (1, 2, 64 * 48, False, "key"),
    (1, 1, 64 * 100 - 17, False, "key"),
    (1, 2, 64 * 64, True, "head"),
    (2, 1, 64 * 64 - 1, True, "key"),
])
def test_segmented_scan(B, H, T, tied, gates):
    w = W[2].scaled(B=B, T=T, H=H, tied=tied, gates=gates)
    _check(w, synth.make_inputs(w, seed=50 + T % 97 + H), 64, ws=True)


def test_segmented_scan_exact_chunks():
    # every chunk flagged for the exact recurrence (query Grams out of range,
    # as in test_large_grams_run_exactly) and a state beyond the fp16 range:
    # the exact path also serves the segment summaries (F without the writes)
    w, inp = _bf16_case(51, T=64 * 48, H=1)
    inp["q"] = inp["q"] * 1024.0
    inp["q_bf16"] = (inp["q_bf16"].astype(np.uint32) + (10 << 7)).astype(np.uint16)
    inp["write"] = inp["write"] * 1000.0
    _check(w, inp, 64, ws=True)
    w, inp = _bf16_case(52, T=64 * 48, H=1)
    inp["S0"] = inp["S0"] * 3.0e5
    _check(w, inp, 64, ws=True)


def test_decode_steps_as_a_replayed_graph():
    # consecutive decode steps captured as one HIP graph (no memset nodes:
    # the step launches one kernel and nothing else) and replayed several
    # times, with eager work and synchronisations between the replays; each
    # replay reproduces the eager steps bit for bit
    import torch
    from gated_delta_rule_decay_amd import recurrent_step

    w = W[4].scaled(B=8, H=4)
    steps = 20
    s0 = torch.from_numpy(synth.make_decode_state(w, seed=71)).cuda()
    inps = [to_device(synth.make_decode_step(w, t, seed=71)) for t in range(steps)]
    state = s0.clone()
    outs = torch.empty((steps, w.B, w.H, w.dv), dtype=torch.float32, device="cuda")

    def run():  # kernel launches only: every step writes its own slice of outs
        for t, d in enumerate(inps):
            recurrent_step(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], state, out=outs[t])

    run()
    torch.cuda.synchronize()
    ref_state, ref_outs = state.clone(), outs.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        state.copy_(s0)
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        run()
    for rep in range(3):
        state.copy_(s0)
        outs.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(state, ref_state) and torch.equal(outs, ref_outs), f"replay {rep}"
        # eager work between replays
        scratch = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        del scratch
