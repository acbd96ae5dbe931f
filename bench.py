"""Throughput of the GDN-2 chunked forward (and of the decode step) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
    python bench.py --summarize DIR      (rocprofv3 CSVs -> profiles/*.txt)

One step is one chunked forward over the whole batch of the full GDN-2
workload (B=8, H=16, T=4096, dk=dv=128, C=64, bf16 q/k/v, fp32 per-channel
decay/erase/write gates and state, S0 ~ N(0, 0.1)), inputs resident in HBM.
``value`` is tokens/s (B*T per step).  The same run also times, each beside
``value`` with its own roofline: the single-pass kernel, o stored as bf16 and
the value-write form on the same inputs; KDA's gates (per-channel decay, one
tied rate per head) on the same shape; the same tokens at sequence lengths
1k..32k (a fixed 32768 tokens per head); the forward on raw inputs (bf16
gate logits, q/k normalised in-kernel); the backward; the same tokens packed
as sequences of mixed lengths; the long-context workload (B=1, T=65536,
two-level scan); the Gated DeltaNet mode (scalar gates, B=4); the recurrent
decode step (256 sequences x 16 heads, fp32 state in HBM updated in place,
1024 consecutive steps with distinct inputs, launched one by one and as one
replayed HIP graph) and the same step on a 1 GiB state; and the fp64 CPU
oracle on the full workload, on the host's cores.

Prints ONE JSON line.  Only one GPU is used; --gpus above 1 exits.

``--plan-out FILE`` records every library call in order (its line, the
number of calls and how many of them were timed), which ``--summarize``
uses to attribute the profiler's dispatches: a call is the run of dispatches
that starts with its first kernel, so the counts alone place every dispatch.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense fp16 / bf16 matrix
PROFILES = os.path.join(ROOT, "profiles")
CHUNK_SOURCES = ("chunk_split.hip", "chunk_common.h", "chunk_mfma.hip", "chunk_general.hip",
                 "kernels.h", "common.h")
DECODE_SOURCES = ("decode.hip", "kernels.h", "common.h")
BWD_SOURCES = ("chunk_bwd.hip", "chunk_bwd_mfma.hip", "kernels.h", "common.h")
CALIB_BYTES = 256 << 20        # the plain device copy that calibrates the byte counters

PLAN: list = []                # every library call of the run, in order


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def plan(label, calls, timed, profile=None):
    """Record `calls` consecutive calls of one line (the last `timed` of
    them timed); `profile` names the traffic summary the line reads."""
    PLAN.append({"label": label, "calls": int(calls), "timed": int(timed), "profile": profile})


def source_hash(names) -> str:
    """Hash of the kernel sources' code: comments and blank lines do not count,
    so a stored counter profile stays valid across comment-only edits."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_delta_rule_decay_amd", "csrc", n)) as f:
            code = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        lines = (re.sub(r"//.*", "", ln).rstrip() for ln in code.splitlines())
        h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()[:16]


# ---- algorithmic bytes and flops ------------------------------------------

def chunk_bytes(w, rate_head=False) -> int:
    """Algorithmic HBM bytes of one chunked forward: every input once, o once,
    S0 read and S_T written once.  ``rate_head``: the decay per key channel,
    the erase / write rates one per token-head (KDA's gates)."""
    e = 2 if w.qkv_dtype == "bf16" else 4
    decay = w.dk * 4 if w.gates == "key" else 4
    rate = 4 if (rate_head or w.gates != "key") else w.dk * 4
    n_rates = 1 if w.tied else 2
    per_tok = (2 * w.dk + w.dv) * e + decay + n_rates * rate + w.dv * 4
    state = w.B * w.H * w.dk * w.dv * 4
    s0 = state if w.s0_std > 0 else 0
    return w.B * w.T * w.H * per_tok + s0 + state


def chunk_flops(w) -> int:
    """Algorithmic flops of one chunked forward, full C x C tiles counted:
    16 C^2 d + 8 C d^2 per chunk-head (untied), 8 C^2 d + 6 C d^2 (tied)."""
    C, d = w.chunk, w.dk
    per_chunk = (8 * C * C * d + 6 * C * d * d) if w.tied else (16 * C * C * d + 8 * C * d * d)
    return w.B * w.H * (w.T // C) * per_chunk


def decode_bytes(w) -> int:
    """Per step: the fp32 state read and written, q/k/v, three per-channel
    fp32 gates and o, for every head."""
    e = 2 if w.qkv_dtype == "bf16" else 4
    per_head = (2 * w.dk + w.dv) * e + 3 * w.dk * 4 + w.dv * 4
    return w.B * w.H * (2 * w.dk * w.dv * 4 + per_head)


def fused_bytes(w) -> int:
    """Algorithmic HBM bytes of one forward with fused input preparation:
    q, k, v bf16, the gate logits bf16, o fp32, S0 and S_T."""
    n_gates = 2 if w.tied else 3
    per_tok = (2 * w.dk + w.dv) * 2 + n_gates * w.dk * 2 + w.dv * 4
    state = w.B * w.H * w.dk * w.dv * 4
    return w.B * w.T * w.H * per_tok + (state if w.s0_std > 0 else 0) + state


def bwd_bytes(w) -> int:
    """Algorithmic HBM bytes of one backward call: the forward's inputs, d_o
    and d_S_T read once; dq, dk, dv, the gate gradients and d_S0 written once
    (fp32)."""
    e = 2 if w.qkv_dtype == "bf16" else 4
    gate = w.dk * 4 if w.gates == "key" else 4
    n_gates = 2 if w.tied else 3
    per_tok = (2 * w.dk + w.dv) * e + n_gates * gate + w.dv * 4 + (2 * w.dk + w.dv) * 4 + n_gates * gate
    state = w.B * w.H * w.dk * w.dv * 4
    return w.B * w.T * w.H * per_tok + 3 * state


def read_traffic(kernel: str, workload: str, src_hash: str):
    """HBM bytes per launch measured with rocprofv3 counters, if the summary
    in profiles/ was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != src_hash:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def roofline_hbm(bytes_alg, ms, traffic=None):
    ach = bytes_alg / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic}


# ---- timing -----------------------------------------------------------------

def time_calls(label, call, steps, warmup, torch, profile=None):
    """`warmup` untimed calls, then `steps` calls timed with HIP events on the
    launch stream (torch's current stream, which the binding passes to the
    library).  Returns wall ms per call, event ms per call, and the median
    and minimum per call."""
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    plan(label, warmup + steps, steps, profile)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    log(f"[bench] timing {steps} calls: {label}")
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        call()
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return {"ms": ms, "kms": ev[0].elapsed_time(ev[steps]) / steps, "med": per[steps // 2], "min": per[0]}


def to_dev(inp, torch):
    out = {}
    for n in ("q", "k", "v"):
        bits = inp.get(n + "_bf16")
        if bits is not None:
            out[n] = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        else:
            out[n] = torch.from_numpy(inp[n]).cuda()
    for n in ("log_decay", "erase", "write", "S0"):
        out[n] = None if inp.get(n) is None else torch.from_numpy(inp[n]).cuda()
    return out


def chunk_line(w, d, label, steps, warmup, torch, *, one_pass=False, value_write=False, out_bf16=False,
               erase=None, tied=None, state0=None, shape=None, profile=None):
    """Time gdn2_chunk_fwd on device inputs `d` (views reshaped to `shape` =
    (B, T) when given), outputs and workspace resident.  Returns the timing
    dict of time_calls."""
    from gated_delta_rule_decay_amd import binding, chunk_fwd

    B, T = shape or (w.B, w.T)
    rs = lambda x: None if x is None else x.reshape((B, T) + tuple(x.shape[2:]))
    q, k, v, la = rs(d["q"]), rs(d["k"]), rs(d["v"]), rs(d["log_decay"])
    eb = rs(d["erase"] if erase is None else erase)
    wr = None if (tied if tied is not None else d["write"] is None) else rs(d["write"])
    s0 = d["S0"] if state0 is None else state0
    o = torch.empty((B, T, w.H, w.dv), dtype=torch.bfloat16 if out_bf16 else torch.float32, device="cuda")
    st = torch.empty((B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    ws = False
    if not one_pass:
        desc = binding._desc_for(q, k, v, la, eb, wr, (B, T, w.H), B, T, w.H, w.chunk, 1.0, value_write, False,
                                 binding.GDN2_BF16 if out_bf16 else binding.GDN2_F32)
        n = binding.chunk_fwd_workspace(desc)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda") if n else False
    kw = dict(chunk=w.chunk, out=o, state_out=st, workspace=ws, value_write=value_write)
    return time_calls(label, lambda: chunk_fwd(q, k, v, la, eb, wr, s0, **kw), steps, warmup, torch, profile)


def line(workload, t, tokens, nbytes, traffic=None, **extra):
    return {"workload": workload, "ms_per_step": round(t["ms"], 4), "kernel_ms": round(t["kms"], 4),
            "kernel_ms_median": round(t["med"], 4), "value": round(tokens / (t["ms"] * 1e-3), 1),
            "unit": "tokens/s", "roofline": roofline_hbm(nbytes, t["kms"], traffic),
            "algorithmic_bytes_per_launch": int(nbytes), **extra}


def decode_inputs(w, n_steps, seed, torch):
    """`n_steps` distinct decode-step inputs drawn on the GPU with the
    workload's distributions (q, k unit-norm rounded to bf16, v ~ N(0, 1)
    bf16, log a = -softplus(N(-2, 1)), b, w = sigmoid(N(0, 1)) fp32)."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    N, H, dk, dv = w.B, w.H, w.dk, w.dv
    rn = lambda *s: torch.randn(s, generator=g, device="cuda", dtype=torch.float32)

    def unit(*s):
        x = rn(*s)
        return (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)

    return {"q": unit(n_steps, N, H, dk), "k": unit(n_steps, N, H, dk), "v": rn(n_steps, N, H, dv).to(torch.bfloat16),
            "log_decay": -torch.nn.functional.softplus(rn(n_steps, N, H, dk) - 2.0),
            "erase": torch.sigmoid(rn(n_steps, N, H, dk)), "write": torch.sigmoid(rn(n_steps, N, H, dk))}


def decode_lines(w, steps, warmup, torch, label, graph=False):
    """Time `steps` consecutive in-place decode steps of workload w, each on
    its own inputs (a pool of `steps` distinct step inputs, or of 64 when the
    pool would not fit comfortably).  With `graph`, also the same steps
    captured as one HIP graph and replayed; the replays must reproduce the
    eager final state and outputs bit for bit."""
    from gated_delta_rule_decay_amd import recurrent_step

    N, H, dk, dv = w.B, w.H, w.dk, w.dv
    per_step = N * H * ((2 * dk + dv) * 2 + 3 * dk * 4)
    pool_n = steps if steps * per_step <= (16 << 30) else 64
    log(f"[bench] decode inputs: {pool_n} distinct steps of {N} x {H} heads")
    inp = decode_inputs(w, pool_n, 4242 + N, torch)
    g0 = torch.Generator(device="cuda").manual_seed(4343 + N)
    s0 = 0.1 * torch.randn((N, H, dk, dv), generator=g0, device="cuda", dtype=torch.float32)
    state = s0.clone()
    o = torch.empty((N, H, dv), dtype=torch.float32, device="cuda")
    call = lambda t: recurrent_step(inp["q"][t % pool_n], inp["k"][t % pool_n], inp["v"][t % pool_n],
                                    inp["log_decay"][t % pool_n], inp["erase"][t % pool_n],
                                    inp["write"][t % pool_n], state, out=o)
    for t in range(warmup):
        call(t)
    torch.cuda.synchronize()
    state.copy_(s0)
    plan(label, warmup + steps, steps, "recurrent_step_" + w.name if N == 256 else None)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {steps} consecutive decode steps: {label}")
    t0 = time.perf_counter()
    ev0.record()
    for t in range(steps):
        call(t)
    ev1.record()
    torch.cuda.synchronize()
    t_eager = {"ms": (time.perf_counter() - t0) * 1e3 / steps, "kms": ev0.elapsed_time(ev1) / steps}
    t_eager["med"] = t_eager["kms"]
    out = {"eager": t_eager, "pool": pool_n}
    if graph:
        ref_state, ref_o = state.clone(), o.clone()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # one untimed step off the capture, as torch asks
            call(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        log(f"[bench] capturing {steps} decode steps as one graph")
        with torch.cuda.graph(g, capture_error_mode="thread_local"):
            for t in range(steps):
                call(t)
        torch.cuda.synchronize()
        # two replays from S0, eager work and a synchronisation between them,
        # each checked against the eager result
        same = True
        for _ in range(2):
            state.copy_(s0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            same = same and bool(torch.equal(state, ref_state)) and bool(torch.equal(o, ref_o))
        plan(label + " (graph: checks)", 2 * steps + 1, 0)
        n_rep = 3
        state.copy_(s0)
        g.replay()  # untimed
        torch.cuda.synchronize()
        ev0.record()
        t0 = time.perf_counter()
        for _ in range(n_rep):
            g.replay()
        ev1.record()
        torch.cuda.synchronize()
        plan(label + " (graph)", (n_rep + 1) * steps, n_rep * steps)
        out["graph"] = {"ms": (time.perf_counter() - t0) * 1e3 / (n_rep * steps),
                        "kms": ev0.elapsed_time(ev1) / (n_rep * steps), "matches_eager": same}
        del g
    del inp, state, s0, o
    return out


# ---- the run ----------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the first dozen calls after an idle period run up to a quarter slower
    # while the GPU's clocks settle; the default warmup covers that
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-extra", action="store_true", help="time only the main workload")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run a plain 256 MiB device copy three times (untimed) whose memory counters "
                         "calibrate the profiler's byte counts")
    ap.add_argument("--no-graph", action="store_true", help="time the decode steps only as single launches")
    ap.add_argument("--plan-out", help="write the order of the library calls here (for --summarize)")
    ap.add_argument("--summarize", metavar="DIR",
                    help="no GPU work: turn the rocprofv3 CSVs under DIR/{trace,fetch,write,mfma} into "
                         "the summaries in profiles/")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(every chain is independent, see the design notes on sharding)", file=sys.stderr)
        sys.exit(2)

    import torch

    from gated_delta_rule_decay_amd import binding, synth

    binding.load_library()  # raises if the HIP library is not built
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    warm = max(1, args.warmup)

    if args.calib_copy:  # before anything else, so its copies are the run's first
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    W = synth.WORKLOADS
    w = W[2]
    chunk_hash = source_hash(CHUNK_SOURCES)
    log(f"[bench] generating {w.name} inputs")
    inp = synth.make_inputs(w, wid=2)
    d = to_dev(inp, torch)
    tm = chunk_line(w, d, w.name, args.steps, warm, torch, profile="chunk_fwd_" + w.name)
    tokens = w.B * w.T
    bytes_alg, flops_alg = chunk_bytes(w), chunk_flops(w)
    result = {
        "metric": "tokens/s for chunked GDN-2 fwd (H=16,dk=dv=128,T=4k) + decode; % roofline",
        "value": round(tokens / (tm["ms"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(tm["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in; f16 MFMA operands, f32 accumulate, f32 state",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: chunked forward B={w.B} H={w.H} T={w.T} "
                               f"dk=dv={w.dk} C={w.chunk}, per-channel decay/erase/write",
                   "global_batch": w.B, "seq_len": w.T, "heads": w.H, "dk": w.dk, "dv": w.dv,
                   "chunk": w.chunk, "parallelism": "single GPU"},
        # the roofline unit is one gdn2_chunk_fwd call (its two kernels):
        # the operation's algorithmic bytes over the HIP-event time of the call
        "roofline": roofline_hbm(bytes_alg, tm["kms"], read_traffic("chunk_fwd", w.name, chunk_hash)),
        "roofline_unit": "one gdn2_chunk_fwd call: chunk_prep_kernel + chunk_scan_kernel",
        "kernel_ms": round(tm["kms"], 4),
        "kernel_ms_median": round(tm["med"], 4),
        "kernel_ms_min": round(tm["min"], 4),
        "algorithmic_bytes_per_launch": bytes_alg,
        "algorithmic_flops_per_launch": flops_alg,
        "mfma_frac_of_algorithmic_flops": round(flops_alg / (tm["kms"] * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
        "chunk_source_hash": chunk_hash,
        "chunk_path": "two-pass: chunk_prep_kernel (every chunk's state-independent products, "
                      "in parallel, into a workspace) then chunk_scan_kernel (the scan over chunks)",
    }
    # the other lines warm up with a third of the main warmup each: the
    # clocks are settled by then, but every line has buffers of its own
    ew = max(1, args.warmup // 3)
    es = max(2, args.steps // 4)
    if not args.no_extra:
        t = chunk_line(w, d, w.name + " (single pass)", es, ew, torch, one_pass=True)
        result["one_pass"] = line(f"{w.name}, single-pass kernel", t, tokens, bytes_alg)
        t = chunk_line(w, d, w.name + " (o stored as bf16)", es, ew, torch, out_bf16=True)
        bo_bytes = bytes_alg - w.B * w.T * w.H * w.dv * 2
        result["bf16_output"] = line(f"{w.name}, o stored as bf16", t, tokens, bo_bytes)
        # the value-write form on the same inputs (dk = dv: the write gate
        # reads as one factor per value channel)
        t = chunk_line(w, d, w.name + " (value-write form)", es, ew, torch, value_write=True)
        result["value_write"] = line(f"{w.name}, value-write form (tied-structure kernels)", t, tokens, bytes_alg)
        # KDA's gates on the same shape: the per-channel decay, one tied rate
        # per token-head (the first channel's erase draw)
        rate = d["erase"][..., 0].contiguous()
        t = chunk_line(w, d, w.name + " (KDA gates)", args.steps, ew, torch, erase=rate, tied=True,
                       profile="chunk_fwd_kda-" + w.name)
        kb = chunk_bytes(w.scaled(tied=True), rate_head=True)
        result["kda"] = line(f"KDA gates on the {w.name} shape: per-channel decay, one tied rate per "
                             f"token-head (two Grams)", t, tokens, kb,
                             read_traffic("chunk_fwd", "kda-" + w.name, chunk_hash),
                             gdn2_over_kda_time=round(tm["kms"] / t["kms"], 3))
        del rate
        # near-flat throughput as the sequence grows: the same 32768 tokens
        # per head as B sequences of T tokens (views of the same inputs)
        g0 = torch.Generator(device="cuda").manual_seed(777)
        s0_all = 0.1 * torch.randn((32, w.H, w.dk, w.dv), generator=g0, device="cuda", dtype=torch.float32)
        sweep = []
        for T in (1024, 2048, 4096, 8192, 16384, 32768):
            B = w.B * w.T // T
            ws_ = w.scaled(B=B, T=T)
            t = chunk_line(ws_, d, f"{w.name} as B={B} T={T}", es, ew, torch, shape=(B, T),
                           state0=s0_all[:B])
            r = line(f"B={B} T={T}", t, tokens, chunk_bytes(ws_))
            sweep.append({"T": T, "B": B, "ms_per_step": r["ms_per_step"], "kernel_ms": r["kernel_ms"],
                          "value": r["value"], "frac": r["roofline"]["frac"]})
        result["seq_len_sweep"] = {"workload": f"{w.name} tokens (32768 per head, H={w.H}) at sequence "
                                               f"length T, B = 32768 / T", "unit": "tokens/s", "points": sweep}
        del s0_all
        result["backward"] = backward_line(w, d, torch, max(2, args.steps // 8), ew)
        result["packed"] = packed_line(w, d, torch, es, ew)
        # one sequence holding most of the tokens: cut into segments of the
        # two-level scan (without them its chain alone would bound the scan)
        result["packed_long"] = packed_line(w, d, torch, es, ew, lengths=[28000, 2000, 1500, 1268])
    del d, inp
    if not args.no_extra:
        # timed like the main line (same steps and warmup), so the two compare
        result["fused_inputs"] = fused_line(w, torch, args.steps, args.warmup, tm["kms"])
        # long context: one sequence per head, T = 65536 (two-level scan)
        w3 = W[3]
        log(f"[bench] generating {w3.name} inputs")
        d3 = to_dev(synth.make_inputs(w3, wid=3), torch)
        t = chunk_line(w3, d3, w3.name, es, ew, torch, profile="chunk_fwd_" + w3.name)
        result["long_context"] = line(f"{w3.name}: B={w3.B} H={w3.H} T={w3.T}, decay spikes", t, w3.B * w3.T,
                                      chunk_bytes(w3), read_traffic("chunk_fwd", w3.name, chunk_hash))
        # its backward: 16 chains, so the state scans run in segments
        result["long_context_backward"] = backward_line(w3, d3, torch, max(2, args.steps // 8), ew)
        del d3
        # Gated DeltaNet mode: scalar gates tied, zero initial state, B=4
        w1 = W[1]
        log(f"[bench] generating {w1.name} inputs")
        d1 = to_dev(synth.make_inputs(w1, wid=1), torch)
        t = chunk_line(w1, d1, w1.name, args.steps, warm, torch, profile="chunk_fwd_" + w1.name)
        result["gdn_mode"] = line(w1.name, t, w1.B * w1.T, chunk_bytes(w1),
                                  read_traffic("chunk_fwd", w1.name, chunk_hash))
        del d1
        # decode: 256 sequences x 16 heads, the state in place, 1024
        # consecutive steps on distinct inputs, launched one by one and as
        # one replayed graph
        w4 = W[4]
        n = args.decode_steps
        dec = decode_lines(w4, n, 3, torch, w4.name, graph=not args.no_graph)
        dh = source_hash(DECODE_SOURCES)
        result["decode"] = line(f"{w4.name}: {w4.B} sequences x H={w4.H}, dk=dv={w4.dk}, fp32 state (256 MiB) in "
                                f"HBM updated in place, {n} consecutive steps, {dec['pool']} distinct step inputs",
                                dec["eager"], w4.B, decode_bytes(w4), read_traffic("recurrent_step", w4.name, dh))
        if "graph" in dec:
            ge = dec["graph"]
            result["decode"]["graph"] = {
                "ms_per_step": round(ge["ms"], 4), "kernel_ms": round(ge["kms"], 4),
                "value": round(w4.B / (ge["ms"] * 1e-3), 1), "unit": "tokens/s",
                "roofline": roofline_hbm(decode_bytes(w4), ge["kms"]),
                "replays_match_eager_bitwise": ge["matches_eager"],
                "what": f"the {n} steps captured as one HIP graph, replayed"}
        # the same step with a 1 GiB state (1024 sequences): beyond the 256 MB
        # Infinity Cache, so every step streams the state from HBM
        w5 = w4.scaled(B=1024, name="gdn2-decode-1gib-bf16")
        dec5 = decode_lines(w5, 256, 3, torch, w5.name)
        result["decode_1gib"] = line(f"{w5.name}: {w5.B} sequences x H={w5.H}, fp32 state (1 GiB) updated in "
                                     f"place, 256 consecutive steps, {dec5['pool']} distinct step inputs",
                                     dec5["eager"], w5.B, decode_bytes(w5))

    if not args.no_cpu:
        from oracle.oracle import available_cores, gdn2_forward

        host = available_cores()
        # the CPU share of this GPU's process (OMP_NUM_THREADS where the
        # machine sets it), and one chain per thread at most
        share = int(os.environ.get("OMP_NUM_THREADS") or host)
        threads = max(1, min(host, share, w.B * w.H))
        log(f"[bench] timing the fp64 oracle on {threads} threads ({host} host cores, share {share})")
        inp = synth.make_inputs(w, wid=2)
        t0 = time.perf_counter()
        gdn2_forward(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"],
                     inp["S0"], threads=threads)
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(tokens / dt, 1), "unit": "tokens/s",
                                  "cores": threads, "host_cores": host, "cpu_share": share, "kind": "oracle",
                                  "sample": f"the whole {w.name} workload ({w.B * w.H} chains x "
                                            f"{w.T} tokens), fp64 token recurrence, one chain per thread, "
                                            f"{dt:.2f} s"}
    if args.plan_out:
        with open(args.plan_out, "w") as f:
            json.dump({"argv": sys.argv[1:], "calib_copy": bool(args.calib_copy), "plan": PLAN,
                       "source_hash": {"chunk_fwd": chunk_hash, "recurrent_step": source_hash(DECODE_SOURCES),
                                       "chunk_bwd": source_hash(BWD_SOURCES)}}, f, indent=1)
    print(json.dumps(result), flush=True)


def backward_line(w, d, torch, steps, warmup):
    """gdn2_chunk_bwd on workload w (random cotangents, workspace resident)."""
    from gated_delta_rule_decay_amd import binding, chunk_bwd

    g = torch.Generator(device="cuda").manual_seed(7)
    d_o = torch.randn((w.B, w.T, w.H, w.dv), device="cuda", generator=g)
    d_st = torch.randn((w.B, w.H, w.dk, w.dv), device="cuda", generator=g)
    desc = binding.make_desc(w.B, w.T, w.H, w.dk, w.dv, w.chunk, binding.GDN2_BF16, 1, 1, 1, w.tied)
    ws = torch.empty(binding.chunk_bwd_workspace(desc), dtype=torch.uint8, device="cuda")
    args = (d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"], d_o, d_st)
    t = time_calls(w.name + " (backward)", lambda: chunk_bwd(*args, chunk=w.chunk, workspace=ws), steps, warmup,
                   torch, "chunk_bwd_" + w.name)
    return line(f"{w.name}: gradients of q, k, v, gates and S0 (fp32 matrix-core kernels: chunk records, state "
                f"and state-gradient scans, per-chunk gradients)", t, w.B * w.T, bwd_bytes(w),
                read_traffic("chunk_bwd", w.name, source_hash(BWD_SOURCES)),
                workspace_bytes=int(ws.numel()))


def packed_line(w, d, torch, steps, warmup, n_seq=12, lengths=None):
    """gdn2_chunk_fwd_varlen on the workload's B*T tokens of every head packed
    as n_seq sequences of drawn lengths (or the lengths given), the same
    q/k/v/gate values, one N(0, 0.1) initial state per sequence."""
    from gated_delta_rule_decay_amd import binding, chunk_fwd_varlen, synth

    tot = w.B * w.T
    drawn = lengths is None
    if drawn:
        lengths = synth.draw_lengths(tot, n_seq, seed=950)
    n_seq = len(lengths)
    flat = lambda x: None if x is None else x.reshape((tot,) + tuple(x.shape[2:]))
    args = [flat(d[n]) for n in ("q", "k", "v", "log_decay", "erase", "write")]
    cu = torch.from_numpy(synth.packed_offsets(lengths)).cuda()
    s0 = torch.from_numpy(synth.make_inputs(w.scaled(B=n_seq, T=1), seed=951)["S0"]).cuda()
    o = torch.empty((tot, w.H, w.dv), dtype=torch.float32, device="cuda")
    st = torch.empty((n_seq, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    desc = binding.make_desc(n_seq, tot, w.H, w.dk, w.dv, w.chunk, binding.GDN2_BF16, 1, 1, 1, False)
    ws = torch.empty(binding.chunk_fwd_varlen_workspace(desc), dtype=torch.uint8, device="cuda")
    kw = dict(chunk=w.chunk, out=o, state_out=st, workspace=ws)
    tag = "packed" if drawn else "packed_long"
    t = time_calls(f"{w.name} ({tag}: {n_seq} sequences)", lambda: chunk_fwd_varlen(*args, cu, s0, **kw), steps,
                   warmup, torch, f"chunk_fwd_{tag}_{w.name}")
    nbytes = chunk_bytes(w.scaled(B=1, T=tot)) + 2 * (n_seq - 1) * w.H * w.dk * w.dv * 4
    return line(f"{w.name} tokens packed as {n_seq} sequences of lengths {lengths} (H={w.H}), two-pass kernels",
                t, tot, nbytes, read_traffic(f"chunk_fwd_{tag}", w.name, source_hash(CHUNK_SOURCES)))


def fused_line(w, torch, steps, warmup, plain_kms):
    """The forward on raw inputs: bf16 gate logits activated and q, k
    L2-normalised inside the kernels (same draws as the main workload);
    `plain_kms` is the main line's event time per call, for the ratio."""
    from gated_delta_rule_decay_amd import binding, chunk_fwd, synth

    log(f"[bench] generating raw {w.name} inputs")
    raw = synth.make_raw_inputs(w, wid=2)
    bf = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = bf(raw["q_bf16"]), bf(raw["k_bf16"]), bf(raw["v_bf16"])
    xa, xb, xw = bf(raw["x_decay_bf16"]), bf(raw["x_erase_bf16"]), bf(raw["x_write_bf16"])
    s0 = torch.from_numpy(raw["S0"]).cuda()
    del raw
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.float32, device="cuda")
    st = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    desc = binding.make_desc(w.B, w.T, w.H, w.dk, w.dv, w.chunk, binding.GDN2_BF16, 1, 1, 1, False,
                             gate_logits=True, qk_l2norm=True)
    ws = torch.empty(binding.chunk_fwd_workspace(desc), dtype=torch.uint8, device="cuda")
    kw = dict(chunk=w.chunk, out=o, state_out=st, workspace=ws, qk_l2norm=True)
    t = time_calls(f"{w.name} (raw inputs)", lambda: chunk_fwd(q, k, v, xa, xb, xw, s0, **kw), steps, warmup,
                   torch, f"chunk_fwd_raw_inputs_{w.name}")
    return line(f"{w.name} on raw inputs: bf16 gate logits (-softplus / sigmoid in-kernel), q and k "
                f"L2-normalised in-kernel", t, w.B * w.T, fused_bytes(w),
                read_traffic("chunk_fwd_raw_inputs", w.name, source_hash(CHUNK_SOURCES)),
                fused_over_plain_time=round(t["kms"] / plain_kms, 3))


# ---- profiles: rocprofv3 CSVs -> profiles/*.txt ------------------------------

def short_name(name: str) -> str:
    """`void gdn2::(anonymous namespace)::k<1, 2>(args...)` -> `k<1, 2>`."""
    n = name.strip()
    if n.startswith("void "):
        n = n[5:]
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):  # the argument list: the first '(' outside <...>
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not n.startswith("(anonymous", i):
            cut = i
            break
    n = n[:cut]
    depth, last = 0, 0
    for i, ch in enumerate(n):  # drop the namespaces (the last '::' outside <...>)
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == ":" and depth == 0 and n[i - 1:i] == ":":
            last = i + 1
    return n[last:]


def _col(row, *names):
    for n in names:
        for k, v in row.items():
            if k and k.strip().lower() == n.lower():
                return v
    raise KeyError(names)


def read_dispatches(d: str):
    """Dispatches of one rocprofv3 run directory, in dispatch order: dicts
    with name, dur_ns (kernel traces) and counters (counter collections)."""
    by_id = {}
    for path in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        for row in csv.DictReader(open(path)):
            i = int(_col(row, "Dispatch_Id"))
            by_id[i] = {"name": _col(row, "Kernel_Name"), "counters": {},
                        "dur_ns": int(_col(row, "End_Timestamp")) - int(_col(row, "Start_Timestamp"))}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(path)):
            i = int(_col(row, "Dispatch_Id"))
            e = by_id.setdefault(i, {"name": _col(row, "Kernel_Name"), "counters": {}, "dur_ns": None})
            c = _col(row, "Counter_Name")
            e["counters"][c] = e["counters"].get(c, 0.0) + float(_col(row, "Counter_Value"))
    return [by_id[i] for i in sorted(by_id)]


def attribute(dispatches, plan_doc):
    """Split the library's dispatches (names in namespace gdn2) into the
    plan's lines and calls: each line's calls all launch the same kernel
    sequence, which starts with the call's first kernel; the distance to that
    kernel's second occurrence is the call's length.  Returns [(line,
    [call, ...])] with each call a list of dispatches."""
    lib = [x for x in dispatches if "gdn2::" in x["name"]]
    for x in lib:
        x["short"] = short_name(x["name"])
    out, i = [], 0
    for ln in plan_doc["plan"]:
        if ln["calls"] < 2 or i >= len(lib):
            raise ValueError(f"line {ln['label']}: needs two calls or more, and dispatches to place")
        first = lib[i]["short"]
        j = i + 1
        while j < len(lib) and lib[j]["short"] != first:
            j += 1
        n_k = j - i
        if i + ln["calls"] * n_k > len(lib):
            raise ValueError(f"line {ln['label']}: fewer dispatches than its calls")
        calls = [lib[i + c * n_k: i + (c + 1) * n_k] for c in range(ln["calls"])]
        seq = [x["short"] for x in calls[0]]
        for c in calls:
            if [x["short"] for x in c] != seq:
                raise ValueError(f"line {ln['label']}: calls launch different kernel sequences")
        out.append((ln, calls))
        i += ln["calls"] * n_k
    if i != len(lib):
        raise ValueError(f"{len(lib) - i} library dispatches left over after the plan")
    return out


def _calibration(dispatches, counter):
    """Median `counter` (KiB) of the run's first three device copies (the
    --calib-copy copies of CALIB_BYTES, issued before anything else)."""
    copies = [x for x in dispatches if "copyBuffer" in x["name"]][:3]
    return statistics.median(x["counters"][counter] for x in copies)


def _header_cmd(sub_dir):
    p = os.path.join(sub_dir, "command.txt")
    return open(p).read().strip() if os.path.exists(p) else "(command.txt missing)"


def summarize(root: str):
    """Write profiles/*.txt from the rocprofv3 runs under `root`: trace/
    (--kernel-trace --stats), fetch/ (--pmc FETCH_SIZE), write/ (--pmc
    WRITE_SIZE), mfma/ (--pmc of the MFMA counters); each holds the plan
    bench.py wrote (plan.json) and the command that ran (command.txt)."""
    os.makedirs(PROFILES, exist_ok=True)
    runs = {}
    for sub in ("trace", "fetch", "write", "mfma"):
        dd = os.path.join(root, sub)
        if os.path.isdir(dd):
            doc = json.load(open(os.path.join(dd, "plan.json")))
            disp = read_dispatches(dd)
            runs[sub] = (dd, doc, disp, attribute(disp, doc))
    if "trace" in runs:
        dd, doc, _, att = runs["trace"]
        lines = ["# rocprofv3 kernel trace, MI355X (gfx950), one GPU: duration per dispatch, by bench line",
                 f"# command (repo root): {_header_cmd(dd)}",
                 "# dispatches are attributed to bench lines by bench.py --summarize from the call plan the run "
                 "wrote (--plan-out); each row covers the line's timed calls only",
                 "line | kernel | timed calls | average_ns | min_ns | max_ns"]
        for ln, calls in att:
            if ln["timed"] == 0:
                continue
            timed = calls[-ln["timed"]:]
            for pos, x in enumerate(timed[0]):
                ds = [c[pos]["dur_ns"] for c in timed]
                lines.append(f"{ln['label']} | {x['short']} | {len(ds)} | {round(sum(ds) / len(ds))} | {min(ds)} | "
                             f"{max(ds)}")
        open(os.path.join(PROFILES, "kernel_stats_all_lines.txt"), "w").write("\n".join(lines) + "\n")
        log("[summarize] wrote profiles/kernel_stats_all_lines.txt")
    if "fetch" in runs and "write" in runs:
        fd, fdoc, fdisp, fatt = runs["fetch"]
        wd, _, wdisp, watt = runs["write"]
        cf, cw = _calibration(fdisp, "FETCH_SIZE"), _calibration(wdisp, "WRITE_SIZE")
        fs, wsc = CALIB_BYTES / 1024 / cf, CALIB_BYTES / 1024 / cw
        for (ln, fcalls), (_, wcalls) in zip(fatt, watt):
            if not ln.get("profile"):
                continue
            prof = ln["profile"]
            kind = next(k for k in ("chunk_fwd", "chunk_bwd", "recurrent_step") if prof.startswith(k))
            names = [x["short"] for x in fcalls[0]]
            fk = sum(statistics.median(c[p]["counters"]["FETCH_SIZE"] for c in fcalls) for p in range(len(names)))
            wk = sum(statistics.median(c[p]["counters"]["WRITE_SIZE"] for c in wcalls) for p in range(len(names)))
            hbm = (fk * fs + wk * wsc) * 1024
            body = [f"# HBM traffic of one call of bench line '{ln['label']}' ({' + '.join(names)}), MI355X, "
                    f"median over the line's {len(fcalls)} calls of each kernel's counter",
                    f"# fetch command: {_header_cmd(fd)}", f"# write command: {_header_cmd(wd)}",
                    f"# calibration: the run's first three copies of {CALIB_BYTES >> 20} MiB (__amd_rocclr_copyBuffer) "
                    f"read FETCH_SIZE {cf:.0f} KiB and WRITE_SIZE {cw:.0f} KiB for {CALIB_BYTES >> 10} KiB each way",
                    f"kernel: {' + '.join(names)}",
                    f"source_hash: {fdoc['source_hash'][kind]}",
                    f"fetch_size_kib: {fk:.0f}", f"write_size_kib: {wk:.0f}",
                    f"fetch_scale: {fs:.4f}", f"write_scale: {wsc:.4f}",
                    f"hbm_bytes_per_launch: {hbm:.0f}"]
            open(os.path.join(PROFILES, f"traffic_{prof}.txt"), "w").write("\n".join(body) + "\n")
            log(f"[summarize] wrote profiles/traffic_{prof}.txt")
    for sub in sorted(os.listdir(root)) if os.path.isdir(root) else []:
        dd = os.path.join(root, sub)
        if sub in ("trace", "fetch", "write", "mfma") or not os.path.exists(os.path.join(dd, "plan.json")):
            continue
        doc = json.load(open(os.path.join(dd, "plan.json")))
        att = attribute(read_dispatches(dd), doc)
        names = sorted({c for _, calls in att for x in calls[0] for c in x["counters"]})
        lines = [f"# rocprofv3 counters per dispatch (median over the line's calls), MI355X (gfx950), one GPU",
                 f"# command (repo root): {_header_cmd(dd)}",
                 "line | kernel | " + " | ".join(names)]
        for ln, calls in att:
            for pos, x in enumerate(calls[0]):
                vals = [statistics.median(cl[pos]["counters"].get(c, 0.0) for cl in calls) for c in names]
                lines.append(f"{ln['label']} | {x['short']} | " + " | ".join(f"{v:.0f}" for v in vals))
        open(os.path.join(PROFILES, f"counters_{sub}.txt"), "w").write("\n".join(lines) + "\n")
        log(f"[summarize] wrote profiles/counters_{sub}.txt")
    if "mfma" in runs:
        dd, _, _, att = runs["mfma"]
        lines = ["# MFMA counters per dispatch (median over the line's calls), MI355X (gfx950), one GPU",
                 f"# command (repo root): {_header_cmd(dd)}",
                 "# executed MFMA flop = SQ_INSTS_VALU_MFMA_MOPS_F16 (resp. _F32) * 512; MFMA busy = "
                 "SQ_VALU_MFMA_BUSY_CYCLES summed over the 1024 SIMDs, divided by GRBM_GUI_ACTIVE of one XCD (the "
                 "counter sums the 8 XCDs, so it is divided by 8): the fraction of SIMD-cycles with the matrix "
                 "core busy",
                 "line | kernel | executed fp16 MFMA GFLOP | executed fp32 MFMA GFLOP | active cycles (per XCD) | "
                 "MFMA busy % of SIMD-cycles"]
        for ln, calls in att:
            for pos, x in enumerate(calls[0]):
                med = lambda c: statistics.median(cl[pos]["counters"].get(c, 0.0) for cl in calls)
                act = med("GRBM_GUI_ACTIVE") / 8
                busy = med("SQ_VALU_MFMA_BUSY_CYCLES")
                lines.append(f"{ln['label']} | {x['short']} | {med('SQ_INSTS_VALU_MFMA_MOPS_F16') * 512 / 1e9:.2f} | "
                             f"{med('SQ_INSTS_VALU_MFMA_MOPS_F32') * 512 / 1e9:.2f} | {act:.0f} | "
                             f"{100 * busy / (1024 * act) if act else 0:.1f}")
        open(os.path.join(PROFILES, "mfma_util_all_lines.txt"), "w").write("\n".join(lines) + "\n")
        log("[summarize] wrote profiles/mfma_util_all_lines.txt")


if __name__ == "__main__":
    main()
