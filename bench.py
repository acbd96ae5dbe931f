"""Throughput of the GDN-2 chunked forward (and of the decode step) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one chunked forward over the whole batch of the full GDN-2
workload (B=8, H=16, T=4096, dk=dv=128, C=64, bf16 q/k/v, fp32 per-channel
decay/erase/write gates and state, S0 ~ N(0, 0.1)), inputs resident in HBM.
``value`` is tokens/s (B*T per step).  The same run also times, each beside
``value`` with its own roofline: the single-pass kernel and the value-write
form on the same inputs, the forward on raw inputs (bf16 gate logits, q/k
normalised in-kernel), the backward, the long-context workload (B=1,
T=65536, two-level scan), the Gated DeltaNet mode (scalar gates, B=4) and
the recurrent decode step (256 sequences x 16 heads, fp32 state in HBM, in
place), and the same tokens packed as sequences of mixed lengths; and the
fp64 CPU oracle on the full workload.

Prints ONE JSON line.  Only one GPU is used; --gpus above 1 exits.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
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


def log(msg):
    print(msg, file=sys.stderr, flush=True)


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


def chunk_bytes(w) -> int:
    """Algorithmic HBM bytes of one chunked forward: every input once, o once,
    S0 read and S_T written once."""
    e = 2 if w.qkv_dtype == "bf16" else 4
    gate = w.dk * 4 if w.gates == "key" else 4
    n_gates = 2 if w.tied else 3
    per_tok = (2 * w.dk + w.dv) * e + n_gates * gate + w.dv * 4
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
    e = 2 if w.qkv_dtype == "bf16" else 4
    per_head = (2 * w.dk + w.dv) * e + 3 * w.dk * 4 + w.dv * 4
    return w.B * w.H * (2 * w.dk * w.dv * 4 + per_head)


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


def time_chunk(w, wid, steps, warmup, torch, chunk_fwd, one_pass=False, inp=None, value_write=False,
               out_bf16=False):
    """Time `steps` chunked forwards of workload w with inputs, outputs and
    the two-pass workspace resident in HBM.  Returns (inputs, wall ms per
    step, HIP-event ms per step on the launch stream)."""
    from gated_delta_rule_decay_amd import binding

    if inp is None:
        log(f"[bench] generating {w.name} inputs")
        inp = synth_make(w, wid)
    d = to_dev(inp, torch)
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.bfloat16 if out_bf16 else torch.float32, device="cuda")
    st = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    ws = False
    if not one_pass:
        desc = binding.make_desc(w.B, w.T, w.H, w.dk, w.dv, w.chunk,
                                 binding.GDN2_BF16 if w.qkv_dtype == "bf16" else binding.GDN2_F32,
                                 int(w.gates == "key"), int(w.gates == "key"), int(w.gates == "key"),
                                 w.tied, form=int(value_write))
        n = binding.chunk_fwd_workspace(desc)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda") if n else False
    args = (d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"])
    kw = dict(chunk=w.chunk, out=o, state_out=st, workspace=ws, value_write=value_write)
    for _ in range(warmup):
        chunk_fwd(*args, **kw)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    log(f"[bench] timing {steps} steps of {w.name}" + (" (one pass)" if one_pass else "")
        + (" (value-write form)" if value_write else ""))
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        chunk_fwd(*args, **kw)
        ev[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    per_call = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    ms_kernel = ev[0].elapsed_time(ev[steps]) / steps
    time_chunk.last = {"kernel_ms_median": round(per_call[steps // 2], 4), "kernel_ms_min": round(per_call[0], 4)}
    return inp, ms_step, ms_kernel


def fused_bytes(w) -> int:
    """Algorithmic HBM bytes of one forward with fused input preparation:
    q, k, v bf16, the gate logits bf16, o fp32, S0 and S_T."""
    n_gates = 2 if w.tied else 3
    per_tok = (2 * w.dk + w.dv) * 2 + n_gates * w.dk * 2 + w.dv * 4
    state = w.B * w.H * w.dk * w.dv * 4
    return w.B * w.T * w.H * per_tok + (state if w.s0_std > 0 else 0) + state


def time_fused(w, torch, chunk_fwd, steps, warmup=1):
    """Time the forward on raw inputs: bf16 gate logits activated and q, k
    L2-normalised inside the kernels (same draws as the main workload)."""
    from gated_delta_rule_decay_amd import binding, synth

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
    for _ in range(warmup):
        chunk_fwd(q, k, v, xa, xb, xw, s0, **kw)
    torch.cuda.synchronize()
    log(f"[bench] timing {steps} steps of {w.name} with fused input preparation")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        chunk_fwd(q, k, v, xa, xb, xw, s0, **kw)
    ev1.record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    kms = ev0.elapsed_time(ev1) / steps
    return {"workload": f"{w.name} on raw inputs: bf16 gate logits (-softplus / sigmoid in-kernel), "
                        f"q and k L2-normalised in-kernel",
            "ms_per_step": round(ms, 4), "kernel_ms": round(kms, 4),
            "value": round(w.B * w.T / (ms * 1e-3), 1), "unit": "tokens/s",
            "roofline": roofline_hbm(fused_bytes(w), kms,
                                     read_traffic("chunk_fwd_raw_inputs", w.name, source_hash(CHUNK_SOURCES))),
            "algorithmic_bytes_per_launch": fused_bytes(w)}


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


def time_backward(w, inp, torch, steps, warmup=1):
    """Time gdn2_chunk_bwd on workload w (random cotangents, workspace
    resident)."""
    from gated_delta_rule_decay_amd import binding, chunk_bwd

    d = to_dev(inp, torch)
    g = torch.Generator(device="cuda").manual_seed(7)
    d_o = torch.randn((w.B, w.T, w.H, w.dv), device="cuda", generator=g)
    d_st = torch.randn((w.B, w.H, w.dk, w.dv), device="cuda", generator=g)
    desc = binding.make_desc(w.B, w.T, w.H, w.dk, w.dv, w.chunk, binding.GDN2_BF16,
                             int(w.gates == "key"), int(w.gates == "key"), int(w.gates == "key"), w.tied)
    ws = torch.empty(binding.chunk_bwd_workspace(desc), dtype=torch.uint8, device="cuda")
    args = (d["q"], d["k"], d["v"], d["log_decay"], d["erase"], d["write"], d["S0"], d_o, d_st)
    for _ in range(warmup):
        chunk_bwd(*args, chunk=w.chunk, workspace=ws)
    torch.cuda.synchronize()
    log(f"[bench] timing {steps} backward calls of {w.name}")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        chunk_bwd(*args, chunk=w.chunk, workspace=ws)
    ev1.record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    k = ev0.elapsed_time(ev1) / steps
    return {"workload": f"{w.name}: gradients of q, k, v, gates and S0 (fp32 matrix-core kernels: chunk "
                        f"records, state and state-gradient scans, per-chunk gradients)",
            "ms_per_step": round(ms, 3), "kernel_ms": round(k, 3),
            "value": round(w.B * w.T / (ms * 1e-3), 1), "unit": "tokens/s",
            "roofline": roofline_hbm(bwd_bytes(w), k, read_traffic("chunk_bwd", w.name, source_hash(BWD_SOURCES))),
            "algorithmic_bytes_per_launch": bwd_bytes(w)}


def time_packed(w, inp, torch, steps, n_seq=12, lengths=None, warmup=1):
    """Time gdn2_chunk_fwd_varlen on the workload's B*T tokens of every head
    packed as n_seq sequences of drawn lengths (or the lengths given: the
    same number of tokens), the same q/k/v/gate values, one N(0, 0.1)
    initial state per sequence."""
    from gated_delta_rule_decay_amd import binding, chunk_fwd_varlen, synth

    tot = w.B * w.T
    if lengths is None:
        lengths = synth.draw_lengths(tot, n_seq, seed=950)
    n_seq = len(lengths)
    d = to_dev(inp, torch)
    flat = lambda x: None if x is None else x.reshape((tot,) + tuple(x.shape[2:]))
    args = [flat(d[n]) for n in ("q", "k", "v", "log_decay", "erase", "write")]
    cu = torch.from_numpy(synth.packed_offsets(lengths)).cuda()
    s0 = torch.from_numpy(synth.make_inputs(w.scaled(B=n_seq, T=1), seed=951)["S0"]).cuda()
    o = torch.empty((tot, w.H, w.dv), dtype=torch.float32, device="cuda")
    st = torch.empty((n_seq, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    desc = binding.make_desc(n_seq, tot, w.H, w.dk, w.dv, w.chunk, binding.GDN2_BF16, 1, 1, 1, False)
    ws = torch.empty(binding.chunk_fwd_varlen_workspace(desc), dtype=torch.uint8, device="cuda")
    kw = dict(chunk=w.chunk, out=o, state_out=st, workspace=ws)
    for _ in range(warmup):
        chunk_fwd_varlen(*args, cu, s0, **kw)
    torch.cuda.synchronize()
    log(f"[bench] timing {steps} packed forwards ({n_seq} sequences)")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        chunk_fwd_varlen(*args, cu, s0, **kw)
    ev1.record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    k = ev0.elapsed_time(ev1) / steps
    nbytes = chunk_bytes(w.scaled(B=1, T=tot)) + 2 * (n_seq - 1) * w.H * w.dk * w.dv * 4
    return {"workload": f"{w.name} tokens packed as {n_seq} sequences of lengths {lengths} "
                        f"(H={w.H}), two-pass kernels",
            "ms_per_step": round(ms, 4), "kernel_ms": round(k, 4),
            "value": round(tot / (ms * 1e-3), 1), "unit": "tokens/s",
            "roofline": roofline_hbm(nbytes, k, read_traffic("chunk_fwd_packed", w.name, source_hash(CHUNK_SOURCES))),
            "algorithmic_bytes_per_launch": nbytes}


def synth_make(w, wid):
    from gated_delta_rule_decay_amd import synth
    return synth.make_inputs(w, wid=wid)


def roofline_hbm(bytes_alg, ms, traffic=None):
    ach = bytes_alg / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the first dozen calls after an idle period run up to a quarter slower
    # while the GPU's clocks settle; the default warmup covers that
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-extra", action="store_true", help="time only the main workload")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (untimed) whose memory counters "
                         "calibrate the profiler's byte counts")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(every chain is independent, see the design notes on sharding)", file=sys.stderr)
        sys.exit(2)

    import torch

    from gated_delta_rule_decay_amd import binding, chunk_fwd, recurrent_step, synth

    binding.load_library()  # raises if the HIP library is not built
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    W = synth.WORKLOADS
    w = W[2]
    inp, ms_step, ms_kernel = time_chunk(w, 2, args.steps, args.warmup, torch, chunk_fwd)
    tokens = w.B * w.T
    value = tokens / (ms_step * 1e-3)
    bytes_alg = chunk_bytes(w)
    flops_alg = chunk_flops(w)
    chunk_hash = source_hash(CHUNK_SOURCES)
    traffic = read_traffic("chunk_fwd", w.name, chunk_hash)
    result = {
        "metric": "tokens/s for chunked GDN-2 fwd (H=16,dk=dv=128,T=4k) + decode; % roofline",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
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
        "roofline": roofline_hbm(bytes_alg, ms_kernel, traffic),
        "roofline_unit": "one gdn2_chunk_fwd call: chunk_prep_kernel + chunk_scan_kernel",
        "kernel_ms": round(ms_kernel, 4),
        **time_chunk.last,
        "algorithmic_bytes_per_launch": bytes_alg,
        "algorithmic_flops_per_launch": flops_alg,
        "mfma_frac_of_algorithmic_flops": round(flops_alg / (ms_kernel * 1e-3) / 1e12
                                                / MFMA_PEAK_TFLOPS, 4),
        "chunk_source_hash": chunk_hash,
        "chunk_path": "two-pass: chunk_prep_kernel (every chunk's state-independent products, "
                      "in parallel, into a workspace) then chunk_scan_kernel (the scan over chunks)",
    }
    # the other lines warm up with a third of the main warmup each: the
    # clocks are settled by then, but every line has buffers of its own
    ew = max(1, args.warmup // 3)
    if not args.no_extra:
        _, ms1p, k1p = time_chunk(w, 2, max(2, args.steps // 4), ew, torch, chunk_fwd, one_pass=True,
                                  inp=inp)
        result["one_pass"] = {"ms_per_step": round(ms1p, 4), "kernel_ms": round(k1p, 4),
                              "value": round(tokens / (ms1p * 1e-3), 1), "unit": "tokens/s"}
        # the value-write form on the same inputs (dk = dv: the write gate
        # reads as one factor per value channel)
        _, msvw, kvw = time_chunk(w, 2, max(2, args.steps // 4), ew, torch, chunk_fwd, inp=inp,
                                  value_write=True)
        # the same call with o stored as bf16 (the fp32 result rounded): o's
        # 512 B per token-head halve
        _, msbo, kbo = time_chunk(w, 2, max(2, args.steps // 4), ew, torch, chunk_fwd, inp=inp, out_bf16=True)
        bo_bytes = chunk_bytes(w) - w.B * w.T * w.H * w.dv * 2
        result["bf16_output"] = {"workload": f"{w.name}, o stored as bf16", "ms_per_step": round(msbo, 4),
                                 "kernel_ms": round(kbo, 4), "value": round(tokens / (msbo * 1e-3), 1),
                                 "unit": "tokens/s", "roofline": roofline_hbm(bo_bytes, kbo),
                                 "algorithmic_bytes_per_launch": bo_bytes}
        result["value_write"] = {"workload": f"{w.name}, value-write form (tied-structure kernels)",
                                 "ms_per_step": round(msvw, 4), "kernel_ms": round(kvw, 4),
                                 "value": round(tokens / (msvw * 1e-3), 1), "unit": "tokens/s",
                                 "roofline": roofline_hbm(chunk_bytes(w), kvw)}
        result["backward"] = time_backward(w, inp, torch, max(2, args.steps // 8), ew)
        result["packed"] = time_packed(w, inp, torch, max(2, args.steps // 4), warmup=ew)
        # one sequence holding most of the tokens: cut into segments of the
        # two-level scan (without them its chain alone would bound the scan)
        result["packed_long"] = time_packed(w, inp, torch, max(2, args.steps // 4),
                                            lengths=[28000, 2000, 1500, 1268], warmup=ew)
    del inp
    if not args.no_extra:
        result["fused_inputs"] = time_fused(w, torch, chunk_fwd, max(2, args.steps // 4), ew)

    if not args.no_extra:
        # long context: one sequence per head, T = 65536 (two-level scan)
        w3 = W[3]
        _, ms3, k3 = time_chunk(w3, 3, max(2, args.steps // 4), ew, torch, chunk_fwd)
        result["long_context"] = {"workload": f"{w3.name}: B={w3.B} H={w3.H} T={w3.T}, decay spikes",
                                  "value": round(w3.B * w3.T / (ms3 * 1e-3), 1), "unit": "tokens/s",
                                  "ms_per_step": round(ms3, 4), "kernel_ms": round(k3, 4),
                                  "roofline": roofline_hbm(chunk_bytes(w3), k3,
                                                           read_traffic("chunk_fwd", w3.name, chunk_hash))}
        # Gated DeltaNet mode: scalar gates tied, zero initial state, B=4
        w1 = W[1]
        _, ms1, k1 = time_chunk(w1, 1, args.steps, args.warmup, torch, chunk_fwd)
        result["gdn_mode"] = {"workload": w1.name, "value": round(w1.B * w1.T / (ms1 * 1e-3), 1),
                              "unit": "tokens/s", "ms_per_step": round(ms1, 4),
                              "roofline": roofline_hbm(chunk_bytes(w1), k1,
                                                       read_traffic("chunk_fwd", w1.name, chunk_hash))}
        # decode: 256 sequences x 16 heads, state in place, a pool of distinct step inputs
        w4 = W[4]
        log("[bench] decode setup")
        state = torch.from_numpy(synth.make_decode_state(w4)).cuda()
        pool = [to_dev(synth.make_decode_step(w4, t), torch) for t in range(8)]
        o4 = torch.empty((w4.B, w4.H, w4.dv), dtype=torch.float32, device="cuda")
        call = lambda d: recurrent_step(d["q"], d["k"], d["v"], d["log_decay"], d["erase"],
                                        d["write"], state, out=o4)
        for t in range(3):
            call(pool[t % len(pool)])
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = args.decode_steps
        t0 = time.perf_counter()
        ev0.record()
        for t in range(n):
            call(pool[t % len(pool)])
        ev1.record()
        torch.cuda.synchronize()
        ms_dec = (time.perf_counter() - t0) * 1e3 / n
        k_dec = ev0.elapsed_time(ev1) / n
        result["decode"] = {
            "workload": f"{w4.name}: {w4.B} sequences x H={w4.H}, dk=dv={w4.dk}, fp32 state "
                        f"in HBM updated in place, {n} consecutive steps",
            "value": round(w4.B / (ms_dec * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(ms_dec, 4), "kernel_ms": round(k_dec, 4),
            "roofline": roofline_hbm(decode_bytes(w4), k_dec,
                                     read_traffic("recurrent_step", w4.name,
                                                  source_hash(DECODE_SOURCES))),
            "algorithmic_bytes_per_launch": decode_bytes(w4),
        }
        del state, pool

    if args.calib_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")  # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = src.numel() * 4
        del src, dst

    if not args.no_cpu:
        from oracle.oracle import available_cores, gdn2_forward

        cores = min(16, available_cores())
        log(f"[bench] timing the fp64 oracle on {cores} threads")
        inp = synth_make(w, 2)
        t0 = time.perf_counter()
        gdn2_forward(inp["q"], inp["k"], inp["v"], inp["log_decay"], inp["erase"], inp["write"],
                     inp["S0"], threads=cores)
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(tokens / dt, 1), "unit": "tokens/s",
                                  "cores": cores, "kind": "oracle",
                                  "sample": f"the whole {w.name} workload ({w.B * w.H} chains x "
                                            f"{w.T} tokens), fp64 token recurrence, {dt:.1f} s"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
