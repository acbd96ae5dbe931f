"""GPU parity of the forward over packed sequences (gdn2_chunk_fwd_varlen).

N sequences of different lengths share one token axis; each is its own
recurrence from its own initial state, so the oracle runs every sequence
alone (gdn2_forward on its slice) and the library's rows and final states are
compared with it.  Covers the two-pass matrix-core kernels (chunks of a
sequence start at its first token; the last one is ragged), the general fp32
kernel, empty sequences, the value-write form and fused input preparation,
the exact path, and at the full GDN-2 size: equal lengths against the
batched forward (bit-exact: the same chunks through the same kernels) and a
drawn length mix on every (sequence, head) chain.  The backward over packed
sequences (gdn2_chunk_bwd_varlen) likewise: every sequence's gradients against
the gradient oracle on that sequence alone (both paths, the value-write form
and fused input preparation), bit-exact against the batched backward at
equal lengths, and at the full size a drawn length mix on every (sequence,
head) chain against the C oracle's reverse pass.
"""
import numpy as np
import pytest

from gated_delta_rule_decay_amd import synth
from oracle.oracle import gdn2_forward, gdn2_forward_raw
from tests.parity_util import MAX_ELEM_FACTOR, TOL_BF16, TOL_F32, chain_errors, rel_l2

pytestmark = pytest.mark.gpu
W = synth.WORKLOADS


def _dev(inp):
    import torch

    def t(x, bits=None):
        if bits is not None:
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()

    d = {n: t(inp[n], inp.get(n + "_bf16")) for n in ("q", "k", "v")}
    for n in ("log_decay", "erase", "write", "x_decay", "x_erase", "x_write"):
        if n in inp:
            d[n] = t(inp[n], inp.get(n + "_bf16"))
    d["S0"] = t(inp["S0"])
    d["cu"] = t(inp["cu_seqlens"])
    return d


def _gates(inp, raw):
    return ("x_decay", "x_erase", "x_write") if raw else ("log_decay", "erase", "write")


def _run(inp, chunk=64, ws=True, raw=False, norm=False, value_write=False, in_place=False):
    import torch
    from gated_delta_rule_decay_amd import chunk_fwd_varlen

    d = _dev(inp)
    ga, gb, gw = (d[n] if n in d else None for n in _gates(inp, raw))
    # the packed tensors as [T, H, d] (the binding also takes [1, T, H, d])
    sq = lambda x: None if x is None else x[0]
    so = d["S0"] if in_place else None
    o, S = chunk_fwd_varlen(sq(d["q"]), sq(d["k"]), sq(d["v"]), sq(ga), sq(gb), sq(gw), d["cu"], d["S0"],
                            chunk=chunk, workspace=ws, value_write=value_write, qk_l2norm=norm,
                            state_out=so)
    torch.cuda.synchronize()
    return o.cpu().numpy(), S.cpu().numpy()


def _oracle_seq(inp, i, h=None, raw=False, norm=False, value_write=False):
    """Oracle on sequence i alone (all heads, or head h): (o [len,H',dv], S [H',dk,dv])."""
    cu = inp["cu_seqlens"]
    lo, hi = int(cu[i]), int(cu[i + 1])
    hs = slice(None) if h is None else slice(h, h + 1)
    s0 = None if inp["S0"] is None else inp["S0"][i:i + 1, hs]
    if hi == lo:  # an empty sequence passes its state through
        return None, s0[0]
    sl = lambda x: None if x is None else x[:, lo:hi, hs]
    g = [sl(inp.get(n)) for n in _gates(inp, raw)]
    if raw:
        o, S = gdn2_forward_raw(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), *g, s0, qk_l2norm=norm,
                                value_write=value_write)
    else:
        o, S = gdn2_forward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), *g, s0, value_write=value_write)
    return o[0], S[0]


def _check(inp, tol, pairs=None, **kw):
    """All sequences (or the (sequence, head) pairs given) against the oracle;
    ``tol`` for o and S, or a pair (o, S)."""
    tol_o, tol_s = tol if isinstance(tol, tuple) else (tol, tol)
    o, S = _run(inp, **kw)
    assert np.isfinite(o).all() and np.isfinite(S).all()
    cu = inp["cu_seqlens"]
    n = len(cu) - 1
    pairs = pairs or [(i, None) for i in range(n)]
    okw = {k: v for k, v in kw.items() if k in ("raw", "norm", "value_write")}
    go, ro, gs, rs = [], [], [], []
    for i, h in pairs:
        o_ref, S_ref = _oracle_seq(inp, i, h, **okw)
        hs = slice(None) if h is None else slice(h, h + 1)
        if o_ref is not None:
            go.append(o[cu[i]:cu[i + 1], hs].ravel())
            ro.append(o_ref.ravel())
        gs.append(S[i, hs].ravel())
        rs.append(S_ref.ravel())
    eo = rel_l2(np.concatenate(go), np.concatenate(ro))
    es = rel_l2(np.concatenate(gs), np.concatenate(rs))
    print(f"  lengths {np.diff(cu).tolist()[:16]} rel_l2 o={eo:.3e} S={es:.3e} (tol {tol_o:.0e}, {tol_s:.0e})",
          flush=True)
    assert eo <= tol_o and es <= tol_s
    return o, S


LENGTHS = [37, 200, 1, 0, 129, 64]  # ragged tails, a one-token and an empty sequence


@pytest.mark.parametrize("ws", [True, False], ids=["two-pass", "general"])
@pytest.mark.parametrize("gates,tied", [("key", False), ("head", True)])
def test_bf16_d128(gates, tied, ws):
    w = W[2].scaled(H=2, gates=gates, tied=tied)
    _check(synth.make_packed_inputs(w, LENGTHS, seed=900), TOL_BF16, ws=ws)


def test_fp32_general_shapes():
    w = W[2].scaled(H=2, dk=48, dv=80, qkv_dtype="f32")
    _check(synth.make_packed_inputs(w, [5, 0, 33, 17, 64], seed=910), TOL_F32, chunk=16)


def test_empty_first_and_last_sequences_in_place():
    # sequences 0 and 3 empty: their states pass through; final states
    # written over the initial ones
    w = W[2].scaled(H=2)
    inp = synth.make_packed_inputs(w, [0, 70, 64, 0], seed=915)
    o, S = _check(inp, TOL_BF16, in_place=True)
    assert np.array_equal(S[0], inp["S0"][0]) and np.array_equal(S[3], inp["S0"][3])


@pytest.mark.parametrize("ws", [True, False], ids=["two-pass", "general"])
def test_value_write_and_fused_inputs(ws):
    w = W[2].scaled(H=2)
    inp = synth.make_packed_inputs(w, [70, 3, 130, 0, 64], seed=920, raw=True)
    _check(inp, TOL_BF16, ws=ws, raw=True, norm=True)
    # the value-write form: a write gate per value channel
    inp = synth.make_packed_inputs(w, [70, 3, 130, 0, 64], seed=925)
    r = np.random.Generator(np.random.PCG64(926))
    inp["write"] = (1 / (1 + np.exp(-r.standard_normal(inp["v"].shape)))).astype(np.float32)
    _check(inp, TOL_BF16, ws=ws, value_write=True)


def test_exact_chunks():
    # a state beyond the fp16 range sends sequence 1's first chunk to the
    # exact fp32 path (rows bounded by its own end): its outputs, dominated by
    # that chunk, come out at the fp32 level; the state decays back into range
    # and the later chunks (and the final state) take the fast path.  The
    # other sequences stay on the fast path throughout.
    w = W[2].scaled(H=2)
    inp = synth.make_packed_inputs(w, [100, 150, 90], seed=930)
    inp["S0"][1] *= 3.0e5
    _check(inp, (1e-5, TOL_BF16), pairs=[(1, None)])
    _check(inp, TOL_BF16, pairs=[(0, None), (2, None)])


@pytest.mark.parametrize("lengths", [[20000, 300, 1000], [1000, 9000, 0, 6000]])
def test_long_sequences_segmented(lengths):
    # sequences of more than L chunks (L = 16 here) are scanned in segments
    # (summaries, then the combine for three or more, then the scan from each
    # segment's entry state); the others in one piece
    w = W[2].scaled(H=2)
    inp = synth.make_packed_inputs(w, lengths, seed=sum(lengths) % 1000)
    _check(inp, TOL_BF16)


def test_segmented_exact_chunks():
    # a long sequence entering with a state beyond the fp16 range: its first
    # segment's chunks run as the exact fp32 recurrence
    w = W[2].scaled(H=1)
    inp = synth.make_packed_inputs(w, [200, 3000, 64], seed=995)
    inp["S0"][1] *= 3.0e5
    _check(inp, (1e-4, TOL_BF16), pairs=[(1, None)])
    _check(inp, TOL_BF16, pairs=[(0, None), (2, None)])


def test_full_size_equal_lengths_match_batched():
    # 8 sequences of 4096 tokens, 16 heads: the packed call runs the same
    # chunks as the batched one through the same kernels (bit-exact)
    import torch
    from gated_delta_rule_decay_amd import chunk_fwd, chunk_fwd_varlen

    w = W[2]
    inp = synth.make_inputs(w, seed=940)
    d = _dev({**inp, "cu_seqlens": synth.packed_offsets([w.T] * w.B)})
    args = [d[n] for n in ("q", "k", "v", "log_decay", "erase", "write")]
    o_b, S_b = chunk_fwd(*args, d["S0"])
    flat = lambda x: x.reshape((w.B * w.T,) + tuple(x.shape[2:]))
    o_p, S_p = chunk_fwd_varlen(*[flat(x) for x in args], d["cu"], d["S0"])
    torch.cuda.synchronize()
    assert torch.equal(flat(o_b), o_p) and torch.equal(S_b, S_p)


def test_full_size_length_mix_every_sequence():
    # 32768 tokens (the GDN-2 workload's 8 x 4096) cut into 12 drawn lengths,
    # 16 heads: every (sequence, head) chain against the oracle run on that
    # sequence alone, per chain (and its largest element error)
    w = W[2]
    lengths = synth.draw_lengths(w.B * w.T, 12, seed=950)
    inp = synth.make_packed_inputs(w, lengths, seed=951)
    o, S = _run(inp)
    cu = inp["cu_seqlens"]
    rel, big = [], []
    for i in range(len(lengths)):
        o_ref, S_ref = _oracle_seq(inp, i)
        parts = [(S[i], S_ref, (1, 2))]
        if o_ref is not None:
            parts.append((o[cu[i]:cu[i + 1]], o_ref, (0, 2)))
        for x, ref, axes in parts:
            assert np.isfinite(x).all()
            r_, m_ = chain_errors(x, ref, axes)
            rel.append(r_)
            big.append(m_)
    rel, big = np.concatenate(rel), np.concatenate(big)
    print(f"  lengths {lengths}: {rel.size} (sequence, head) checks of o and S, worst rel_l2 {rel.max():.3e}, "
          f"largest element error {big.max():.3e} x chain RMS", flush=True)
    assert rel.max() <= TOL_BF16 and big.max() <= MAX_ELEM_FACTOR * TOL_BF16


# ---- the backward over packed sequences ------------------------------------

def _bwd_check(inp, seed, raw=False, vw=False, chunk=64, pairs=None):
    """Gradients of every sequence (or of the (sequence, head) pairs given)
    against the gradient oracle run on that sequence alone."""
    import torch
    from gated_delta_rule_decay_amd import chunk_bwd_varlen
    from oracle.oracle_bwd import gdn2_backward

    r = np.random.Generator(np.random.PCG64(seed))
    cu = inp["cu_seqlens"]
    n = len(cu) - 1
    d_o = r.standard_normal(inp["v"].shape).astype(np.float32)
    d_st = r.standard_normal(inp["S0"].shape).astype(np.float32)
    d = _dev(inp)
    gn = _gates(inp, raw)
    sq = lambda x: None if x is None else x[0]
    g = chunk_bwd_varlen(sq(d["q"]), sq(d["k"]), sq(d["v"]), *[sq(d.get(x)) for x in gn], d["cu"], d["S0"],
                         torch.from_numpy(d_o[0]).cuda(), torch.from_numpy(d_st).cuda(), chunk=chunk,
                         value_write=vw, qk_l2norm=raw)
    torch.cuda.synchronize()
    got = {k: (None if x is None else x.cpu().numpy()) for k, x in g.items()}
    names = ("dq", "dk", "dv", "d_log_decay", "d_erase", "d_write", "d_state0")
    acc = {k: ([], []) for k in names}
    for i, h in pairs or [(i, None) for i in range(n)]:
        lo, hi = int(cu[i]), int(cu[i + 1])
        hs = slice(None) if h is None else slice(h, h + 1)
        if hi > lo:
            sl = lambda x: None if x is None else x[:, lo:hi, hs]
            ref = gdn2_backward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), *[sl(inp.get(x)) for x in gn],
                                inp["S0"][i:i + 1, hs], sl(d_o), d_st[i:i + 1, hs], value_write=vw, raw=raw)
        for key in names:
            if got[key] is None:
                continue
            if key == "d_state0":
                want = ref[key][0] if hi > lo else d_st[i, hs]
                acc[key][0].append(got[key][i, hs].ravel())
                acc[key][1].append(np.asarray(want).ravel())
            elif hi > lo:
                acc[key][0].append(got[key][lo:hi, hs].ravel())
                acc[key][1].append(ref[key][0].ravel())
    errs = {k: rel_l2(np.concatenate(a), np.concatenate(b)) for k, (a, b) in acc.items() if a}
    print("  " + " ".join(f"{k}={e:.1e}" for k, e in errs.items()), flush=True)
    for k, e in errs.items():
        assert e <= TOL_F32, (k, e)


@pytest.mark.parametrize("gates,tied", [("key", False), ("head", True)])
def test_backward_bf16_d128(gates, tied):
    w = W[2].scaled(H=2, gates=gates, tied=tied)
    _bwd_check(synth.make_packed_inputs(w, LENGTHS, seed=960), seed=961)


def test_backward_general_shapes():
    w = W[2].scaled(H=2, dk=48, dv=80, qkv_dtype="f32")
    _bwd_check(synth.make_packed_inputs(w, [5, 0, 33, 17, 64], seed=970), seed=971, chunk=16)


def test_backward_raw_inputs_value_write():
    w = W[2].scaled(H=2)
    inp = synth.make_packed_inputs(w, [70, 3, 130, 0, 64], seed=980, raw=True)
    r = np.random.Generator(np.random.PCG64(981))
    inp["x_write"], inp["x_write_bf16"] = synth.round_to_bf16(r.standard_normal(inp["v"].shape).astype(np.float32))
    _bwd_check(inp, seed=982, raw=True, vw=True)


def test_backward_full_size_equal_lengths_match_batched():
    # 8 x 4096 tokens, 16 heads: the same chunks through the same kernels as
    # the batched backward (bit-exact)
    import torch
    from gated_delta_rule_decay_amd import chunk_bwd, chunk_bwd_varlen

    w = W[2]
    inp = synth.make_inputs(w, seed=990)
    d = _dev({**inp, "cu_seqlens": synth.packed_offsets([w.T] * w.B)})
    gen = torch.Generator(device="cuda").manual_seed(991)
    d_o = torch.randn((w.B, w.T, w.H, w.dv), device="cuda", generator=gen)
    d_st = torch.randn((w.B, w.H, w.dk, w.dv), device="cuda", generator=gen)
    args = [d[n] for n in ("q", "k", "v", "log_decay", "erase", "write")]
    gb = chunk_bwd(*args, d["S0"], d_o, d_st)
    flat = lambda x: x.reshape((w.B * w.T,) + tuple(x.shape[2:]))
    gp = chunk_bwd_varlen(*[flat(x) for x in args], d["cu"], d["S0"], flat(d_o), d_st)
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv", "d_log_decay", "d_erase", "d_write"):
        assert torch.equal(flat(gb[key]), gp[key]), key
    assert torch.equal(gb["d_state0"], gp["d_state0"])


def test_backward_full_size_length_mix_every_sequence():
    # the GDN-2 workload's 32768 tokens cut into 12 drawn lengths, 16 heads:
    # every (sequence, head) chain's gradients against the C oracle's reverse
    # pass on that sequence alone, per chain (ragged last chunks, and the
    # scans' and gradient kernel's chain mapping over packed sequences)
    import torch
    from gated_delta_rule_decay_amd import chunk_bwd_varlen
    from oracle.oracle import gdn2_backward_c
    from tests.parity_util import check_every_chain

    w = W[2]
    lengths = synth.draw_lengths(w.B * w.T, 12, seed=950)
    inp = synth.make_packed_inputs(w, lengths, seed=955)
    cu = inp["cu_seqlens"]
    r = np.random.Generator(np.random.PCG64(956))
    d_o = r.standard_normal(inp["v"].shape).astype(np.float32)
    d_st = r.standard_normal(inp["S0"].shape).astype(np.float32)
    d = _dev(inp)
    gn = _gates(inp, False)
    sq = lambda x: None if x is None else x[0]
    g = chunk_bwd_varlen(sq(d["q"]), sq(d["k"]), sq(d["v"]), *[sq(d.get(x)) for x in gn], d["cu"], d["S0"],
                         torch.from_numpy(d_o[0]).cuda(), torch.from_numpy(d_st).cuda())
    torch.cuda.synchronize()
    got = {k: (None if x is None else x.cpu().numpy()) for k, x in g.items()}
    names = ("dq", "dk", "dv", "d_log_decay", "d_erase", "d_write")
    for i in range(len(lengths)):
        lo, hi = int(cu[i]), int(cu[i + 1])
        if hi == lo:  # an empty sequence passes its state gradient through
            assert np.array_equal(got["d_state0"][i], d_st[i])
            continue
        sl = lambda x: None if x is None else x[:, lo:hi]
        ref = gdn2_backward_c(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), *[sl(inp.get(x)) for x in gn],
                              inp["S0"][i:i + 1], sl(d_o), d_st[i:i + 1])
        tensors = [(n, got[n][lo:hi], ref[n][0], (0, 2)) for n in names if got[n] is not None]
        tensors.append(("d_state0", got["d_state0"][i], ref["d_state0"][0], (1, 2)))
        check_every_chain(f"packed backward, sequence {i} ({hi - lo} tokens)", tensors, TOL_F32)
