"""Seeded synthetic workloads for the gated delta rule-2 token mixer.

This module only draws inputs.  It holds none of the recurrence's arithmetic,
so both the fp64 oracle (test side) and the GPU library (product side) can
consume exactly the same values without sharing any computation.

Recipe (numpy ``Generator(PCG64(seed))``, default ``seed = 20261203 + id``):

* draw order: q, k, v, x_a, x_b, x_w, S0, spikes;
* q, k ~ N(0, 1), L2-normalised over the key channels of each token-head in
  fp64 (the pages use normalised keys for stability: course slides,
  "Stability"), then cast to fp32, then rounded to bf16 (round to nearest
  even) when the workload's q/k/v dtype is bf16;
* v ~ N(0, 1), cast the same way;
* decay: log a = -softplus(x_a), x_a ~ N(-2, 1), so a = exp(log a) lies in
  (0, 1) as the pages require of the decay gate ("Gated DeltaNet" page,
  gate alpha in (0, 1)); erase b = sigmoid(x_b), write w = sigmoid(x_w),
  x_b, x_w ~ N(0, 1) (sigmoid-like gates, same page, "Read the limiting
  cases"); every gate is stored as fp32;
* S0 ~ N(0, 0.1) (standard deviation 0.1) where the workload has a nonzero
  initial state;
* long-context spikes: at every token t with t % 4096 == 0, 13 of 128 key
  channels (10 %, rounded), chosen per (batch, head, spike) without
  replacement, get a fresh x_a ~ N(+6, 0.5): a near-zero decay that resets
  those channels.

The oracle reads the stored fp32 / bf16-exact values, so rounding to bf16 is
part of the input, never a source of disagreement.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

BASE_SEED = 20261203


@dataclass(frozen=True)
class Workload:
    """One synthetic workload shape and distribution."""

    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int
    qkv_dtype: str  # "f32" or "bf16"
    gates: str  # "key": per key channel decay/erase/write; "head": scalar per token-head
    tied: bool  # write gate tied to the erase gate
    s0_std: float  # 0.0: zero initial state
    spikes: bool = False
    decode_steps: int = 0  # > 0: a recurrent-decode workload (T is 1 per step)
    extra: dict = field(default_factory=dict)

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def tokens(self) -> int:
        if self.decode_steps:
            return self.B * self.decode_steps
        return self.B * self.T


# The five workloads: a tiny fp32 case, the Gated DeltaNet mode, full GDN-2,
# long context with decay spikes, and recurrent decode.
WORKLOADS = {
    0: Workload("tiny-gdn2-fp32", B=1, H=2, T=256, dk=32, dv=32, chunk=16,
                qkv_dtype="f32", gates="key", tied=False, s0_std=0.0),
    1: Workload("gdn-scalar-gates-bf16", B=4, H=16, T=4096, dk=128, dv=128, chunk=64,
                qkv_dtype="bf16", gates="head", tied=True, s0_std=0.0),
    2: Workload("gdn2-bf16", B=8, H=16, T=4096, dk=128, dv=128, chunk=64,
                qkv_dtype="bf16", gates="key", tied=False, s0_std=0.1),
    3: Workload("gdn2-long-bf16", B=1, H=16, T=65536, dk=128, dv=128, chunk=64,
                qkv_dtype="bf16", gates="key", tied=False, s0_std=0.1, spikes=True),
    4: Workload("gdn2-decode-bf16", B=256, H=16, T=1, dk=128, dv=128, chunk=64,
                qkv_dtype="bf16", gates="key", tied=False, s0_std=0.1,
                decode_steps=1024),
}


def round_to_bf16(x: np.ndarray):
    """Round fp32 values to bf16 with round-to-nearest-even.

    Returns (values as float32 holding the exact bf16 numbers, raw uint16
    bf16 bit patterns).  Finite inputs only.
    """
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    u = x32.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    bits = (r >> np.uint32(16)).astype(np.uint16)
    return r.view(np.float32), bits


def _softplus(x: np.ndarray) -> np.ndarray:
    """log(1 + exp(x)) in fp64 without overflow."""
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, 1e-30)


def _cast_qkv(x64: np.ndarray, dtype: str) -> dict:
    x32 = x64.astype(np.float32)
    if dtype == "bf16":
        vals, bits = round_to_bf16(x32)
        return {"values": vals, "bf16_bits": bits}
    return {"values": x32, "bf16_bits": None}


def _gates(rng, shape_tok, dk, kind):
    gshape = shape_tok + ((dk,) if kind == "key" else ())
    x_a = rng.normal(-2.0, 1.0, size=gshape)
    x_b = rng.normal(0.0, 1.0, size=gshape)
    x_w = rng.normal(0.0, 1.0, size=gshape)
    return x_a, x_b, x_w


def make_inputs(w: Workload, seed: int | None = None, wid: int | None = None) -> dict:
    """Draw one chunked-forward workload.

    Returns a dict with float32 arrays ``q, k, v`` ([B,T,H,d]; exact bf16
    values when ``qkv_dtype == "bf16"``, with the raw bits in
    ``q_bf16`` / ``k_bf16`` / ``v_bf16``), ``log_decay``, ``erase``,
    ``write`` (None when tied) shaped [B,T,H,dk] or [B,T,H], and ``S0``
    ([B,H,dk,dv] float32, or None for a zero initial state).
    """
    if seed is None:
        seed = BASE_SEED + (wid if wid is not None else 0)
    rng = np.random.Generator(np.random.PCG64(seed))
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    q64 = _normalise(rng.normal(0.0, 1.0, size=(B, T, H, dk)))
    k64 = _normalise(rng.normal(0.0, 1.0, size=(B, T, H, dk)))
    v64 = rng.normal(0.0, 1.0, size=(B, T, H, dv))
    x_a, x_b, x_w = _gates(rng, (B, T, H), dk, w.gates)
    s0 = None
    if w.s0_std > 0.0:
        s0 = rng.normal(0.0, w.s0_std, size=(B, H, dk, dv)).astype(np.float32)
    if w.spikes:
        assert w.gates == "key"
        n_sp = int(round(0.1 * dk))
        for t0 in range(0, T, 4096):
            for b in range(B):
                for h in range(H):
                    ch = rng.choice(dk, size=n_sp, replace=False)
                    x_a[b, t0, h, ch] = rng.normal(6.0, 0.5, size=n_sp)
    out = {}
    for name, x in (("q", q64), ("k", k64), ("v", v64)):
        c = _cast_qkv(x, w.qkv_dtype)
        out[name] = c["values"]
        out[name + "_bf16"] = c["bf16_bits"]
    out["log_decay"] = (-_softplus(x_a)).astype(np.float32)
    out["erase"] = _sigmoid(x_b).astype(np.float32)
    out["write"] = None if w.tied else _sigmoid(x_w).astype(np.float32)
    out["S0"] = s0
    return out


def make_raw_inputs(w: Workload, seed: int | None = None, wid: int | None = None) -> dict:
    """The same draws as ``make_inputs`` before any input preparation: q, k
    ~ N(0, 1) NOT normalised, and the gate logits x_a, x_b, x_w themselves,
    rounded to bf16 (bits in ``*_bf16``, exact values as fp32 arrays).

    Returns q, k, v (+ ``_bf16`` bits), ``x_decay``, ``x_erase``, ``x_write``
    (None when tied) shaped [B,T,H,dk] or [B,T,H] (+ ``_bf16`` bits), and S0.
    """
    if seed is None:
        seed = BASE_SEED + (wid if wid is not None else 0)
    rng = np.random.Generator(np.random.PCG64(seed))
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    q64 = rng.normal(0.0, 1.0, size=(B, T, H, dk))
    k64 = rng.normal(0.0, 1.0, size=(B, T, H, dk))
    v64 = rng.normal(0.0, 1.0, size=(B, T, H, dv))
    x_a, x_b, x_w = _gates(rng, (B, T, H), dk, w.gates)
    s0 = None
    if w.s0_std > 0.0:
        s0 = rng.normal(0.0, w.s0_std, size=(B, H, dk, dv)).astype(np.float32)
    out = {}
    for name, x in (("q", q64), ("k", k64), ("v", v64)):
        c = _cast_qkv(x, w.qkv_dtype)
        out[name] = c["values"]
        out[name + "_bf16"] = c["bf16_bits"]
    for name, x in (("x_decay", x_a), ("x_erase", x_b), ("x_write", None if w.tied else x_w)):
        if x is None:
            out[name], out[name + "_bf16"] = None, None
            continue
        vals, bits = round_to_bf16(x.astype(np.float32))
        out[name], out[name + "_bf16"] = vals, bits
    out["S0"] = s0
    return out


def packed_offsets(lengths) -> np.ndarray:
    """int32 offsets [N+1] of sequences of the given lengths packed in order."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def draw_lengths(total: int, n: int, seed: int) -> list[int]:
    """A length mix for packed sequences: ``n`` lengths summing to ``total``,
    the shares drawn as Exp(1) weights (a uniform Dirichlet split: a few long
    documents and many short ones, zeros possible), cut points rounded down."""
    r = np.random.Generator(np.random.PCG64(seed))
    wts = r.exponential(1.0, size=n)
    cuts = np.floor(total * np.cumsum(wts) / wts.sum()).astype(np.int64)
    cuts[-1] = total
    return np.diff(np.concatenate([[0], cuts])).tolist()


def make_packed_inputs(w: Workload, lengths, seed: int, raw: bool = False) -> dict:
    """Inputs for N = len(lengths) sequences packed along one token axis:
    the workload recipe drawn for B = 1 and T = sum(lengths) (``raw``: before
    input preparation, as ``make_raw_inputs``), one initial state per
    sequence from the recipe's S0 draw with B = N (seed + 1), and the
    offsets ``cu_seqlens``."""
    T = int(sum(lengths))
    gen = make_raw_inputs if raw else make_inputs
    out = gen(w.scaled(B=1, T=T), seed=seed)
    out["S0"] = gen(w.scaled(B=len(lengths), T=1), seed=seed + 1)["S0"]
    out["cu_seqlens"] = packed_offsets(lengths)
    return out


def make_decode_state(w: Workload, seed: int | None = None) -> np.ndarray:
    """Initial fp32 state [N,H,dk,dv] ~ N(0, s0_std) for a decode workload."""
    if seed is None:
        seed = BASE_SEED + 4
    rng = np.random.Generator(np.random.PCG64([seed, 0xD0]))
    return rng.normal(0.0, w.s0_std, size=(w.B, w.H, w.dk, w.dv)).astype(np.float32)


def make_decode_step(w: Workload, step: int, seed: int | None = None) -> dict:
    """Inputs of decode step ``step`` for all N sequences, drawn as the chunked
    workloads draw one token: q, k, v [N,H,d]; gates [N,H,dk] or [N,H]."""
    if seed is None:
        seed = BASE_SEED + 4
    rng = np.random.Generator(np.random.PCG64([seed, 1 + step]))
    N, H, dk, dv = w.B, w.H, w.dk, w.dv
    q64 = _normalise(rng.normal(0.0, 1.0, size=(N, H, dk)))
    k64 = _normalise(rng.normal(0.0, 1.0, size=(N, H, dk)))
    v64 = rng.normal(0.0, 1.0, size=(N, H, dv))
    x_a, x_b, x_w = _gates(rng, (N, H), dk, w.gates)
    out = {}
    for name, x in (("q", q64), ("k", k64), ("v", v64)):
        c = _cast_qkv(x, w.qkv_dtype)
        out[name] = c["values"]
        out[name + "_bf16"] = c["bf16_bits"]
    out["log_decay"] = (-_softplus(x_a)).astype(np.float32)
    out["erase"] = _sigmoid(x_b).astype(np.float32)
    out["write"] = None if w.tied else _sigmoid(x_w).astype(np.float32)
    return out
