"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the library through its binding, run the oracle on the same values, and
compare with the relative L2 error over a whole tensor (accumulated in fp64).
"""
from __future__ import annotations

import numpy as np

from gated_delta_rule_decay_amd import synth
from oracle.oracle import gdn2_forward

TOL_F32 = 1e-5   # relative L2, fp32 q/k/v
TOL_BF16 = 2e-3  # relative L2, bf16 q/k/v


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def to_device(inp: dict, device="cuda"):
    """numpy workload dict -> torch tensors on the GPU (bf16 from the raw bits)."""
    import torch

    out = {}
    for name in ("q", "k", "v"):
        bits = inp.get(name + "_bf16")
        if bits is not None:
            t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(inp[name], dtype=np.float32))
        out[name] = t.to(device)
    for name in ("log_decay", "erase", "write", "S0"):
        x = inp.get(name)
        out[name] = None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(device)
    return out


def gpu_chunk(inp: dict, chunk: int, **kw):
    import torch
    from gated_delta_rule_decay_amd import chunk_fwd

    d = to_device(inp)
    o, S = chunk_fwd(d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"],
                     chunk=chunk, **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), S.cpu().numpy()


def oracle_chunk(inp: dict, chains=None, q_scale=1.0):
    """Oracle on all chains, or on the (b, h) pairs listed in ``chains``."""
    if chains is None:
        return gdn2_forward(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"],
                            inp["write"], inp["S0"], q_scale=q_scale)
    outs_o, outs_S = [], []
    for b, h in chains:
        sl = lambda x: None if x is None else x[b:b + 1, :, h:h + 1]
        s0 = None if inp["S0"] is None else inp["S0"][b:b + 1, h:h + 1]
        o, S = gdn2_forward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["log_decay"]),
                            sl(inp["erase"]), sl(inp["write"]), s0, q_scale=q_scale)
        outs_o.append(o[0, :, 0])
        outs_S.append(S[0, 0])
    return np.stack(outs_o), np.stack(outs_S)


def pick_chains(w: synth.Workload, n: int, seed: int = 0):
    r = np.random.Generator(np.random.PCG64(seed))
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    idx = r.choice(len(pairs), size=min(n, len(pairs)), replace=False)
    return [pairs[i] for i in sorted(idx)]


# An error confined to a few outputs hardly moves a relative L2 norm over a
# whole chain.  Besides the rel-L2 bound, each chain's largest element error,
# relative to the chain's RMS, is bounded by MAX_ELEM_FACTOR times the
# tolerance (measured rel-L2 sits well below the tolerance, and the largest
# of ~5e5 roughly Gaussian element errors is about 5 of their RMS), so a
# single wholly wrong element -- an error of the order of the RMS itself --
# fails the check.
MAX_ELEM_FACTOR = 10.0


def chain_errors(x, ref, chain_axes):
    """Per-chain relative L2 error of ``x`` against ``ref`` and per-chain
    largest |x - ref| relative to the chain's RMS of ``ref``; the chain is
    what ``chain_axes`` (the within-chain axes) sum over."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = x - ref
    num = np.sqrt((d * d).sum(axis=chain_axes))
    den = np.sqrt((ref * ref).sum(axis=chain_axes))
    count = int(np.prod([ref.shape[a] for a in chain_axes]))
    safe = np.where(den > 0, den, 1.0)
    rel = np.where(den > 0, num / safe, num)
    mx = np.abs(d).max(axis=chain_axes) / np.where(den > 0, safe / np.sqrt(count), 1.0)
    return rel, mx


def check_every_chain(label, tensors, tol):
    """Assert, for every (name, x, ref, chain_axes) in ``tensors``, that x is
    finite, that the whole tensor and every chain meet the relative-L2
    tolerance, and that no chain's largest element error exceeds
    MAX_ELEM_FACTOR * tol times its RMS.  Prints the worst chain of each."""
    for name, x, ref, axes in tensors:
        assert np.isfinite(np.asarray(x)).all(), f"{label} {name}: non-finite values"
        rel, mx = chain_errors(x, ref, axes)
        overall = rel_l2(x, ref)
        worst = tuple(int(i) for i in np.unravel_index(int(np.argmax(rel)), rel.shape))
        print(f"  {label} {name}: {rel.size} chains, rel_l2 overall {overall:.3e}, worst chain "
              f"{worst} {rel.max():.3e}, largest element error {mx.max():.3e} x chain RMS", flush=True)
        assert overall <= tol, f"{label} {name}: overall rel_l2 {overall:.3e} > {tol:.0e}"
        assert rel.max() <= tol, f"{label} {name}: chain {worst} rel_l2 {rel.max():.3e} > {tol:.0e}"
        assert mx.max() <= MAX_ELEM_FACTOR * tol, (
            f"{label} {name}: an element error of {mx.max():.3e} x chain RMS "
            f"(bound {MAX_ELEM_FACTOR * tol:.0e})")
