"""TEST INFRASTRUCTURE ONLY -- Python loader for the fp64 CPU oracle.

The oracle (``gdn2_oracle.c`` beside this file) is the plain token-by-token
definition of the gated delta rule-2 recurrence in fp64.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this module.  The GPU library never imports, links or calls it, and
this module imports nothing from the GPU package.

The operation, per (batch, head) chain with state S (dk x dv, key-by-value):
decay S <- Diag(a_t) S, read m = S^T k_t, then
S <- S - (b_t*k_t) m^T + (w_t*k_t) v_t^T, then o_t = S^T (q_scale q_t)
("Gated DeltaNet-2" blog summary, "Core Mechanism"; "Gated DeltaNet" page,
"Decay first, then compute the write error"; course slides, "Worked case --
full trace").
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn2_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            dp = ctypes.POINTER(ctypes.c_double)
            i64 = ctypes.c_int64
            lib.gdn2_oracle_fwd.restype = ctypes.c_int
            lib.gdn2_oracle_fwd.argtypes = [
                i64, i64, i64, i64, i64,
                dp, dp, dp,
                dp, ctypes.c_int,
                dp, ctypes.c_int,
                dp, ctypes.c_int,
                dp, ctypes.c_double,
                dp, dp, ctypes.c_int, ctypes.c_int,
            ]
            lib.gdn2_oracle_bwd.restype = ctypes.c_int
            lib.gdn2_oracle_bwd.argtypes = [
                i64, i64, i64, i64, i64,
                dp, dp, dp,
                dp, ctypes.c_int,
                dp, ctypes.c_int,
                dp, ctypes.c_int,
                dp, ctypes.c_double,
                dp, dp,
                dp, dp, dp, dp, dp, dp, dp,
                ctypes.c_int, ctypes.c_int,
            ]
            lib.gdn2_oracle_max_threads.restype = ctypes.c_int
            lib.gdn2_oracle_max_threads.argtypes = []
            _lib = lib
    return _lib


def available_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def gdn2_forward(q, k, v, log_decay, erase, write=None, S0=None, q_scale=1.0,
                 threads: int | None = None, value_write=False):
    """Run the recurrence token by token in fp64.

    Shapes: q, k [B,T,H,dk]; v [B,T,H,dv]; each gate either [B,T,H,dk]
    (one value per key channel) or [B,T,H] (one per token-head); S0
    [B,H,dk,dv] or None (zeros); write None ties it to erase.
    ``value_write``: the gist.science form (write gate per value channel,
    [B,T,H,dv] or [B,T,H], required; the erase gate weights the read).
    Returns (o [B,T,H,dv], S_T [B,H,dk,dv]) as float64 arrays.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, dk = k.shape
    dv = v.shape[3]
    assert q.shape == k.shape and v.shape[:3] == (B, T, H)
    la, b, w, s0 = _f64(log_decay), _f64(erase), _f64(write), _f64(S0)

    def kind(g, d=dk):
        if g.shape == (B, T, H, d):
            return 1
        if g.shape == (B, T, H):
            return 0
        raise ValueError(f"gate shape {g.shape} is neither [B,T,H,{d}] nor [B,T,H]")

    la_k, b_k = kind(la), kind(b)
    if value_write and w is None:
        raise ValueError("the value-write form needs a write gate")
    w_k = kind(w, dv if value_write else dk) if w is not None else 0
    if s0 is not None:
        assert s0.shape == (B, H, dk, dv)
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    S_T = np.zeros((B, H, dk, dv), dtype=np.float64)
    nthreads = threads or available_cores()
    rc = _load().gdn2_oracle_fwd(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(la), la_k, _ptr(b), b_k, _ptr(w), w_k,
                                 _ptr(s0), float(q_scale), _ptr(o), _ptr(S_T),
                                 1 if value_write else 0, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    return o, S_T


def gdn2_backward_c(q, k, v, log_decay, erase, write=None, S0=None, d_o=None, d_state=None,
                    q_scale=1.0, threads: int | None = None):
    """Gradients of L = <d_o, o> + <d_state, S_T> with respect to every input
    of ``gdn2_forward`` (key form), by the reverse pass written out by hand in
    ``gdn2_oracle.c`` (fp64, chains in parallel).  Same arguments and the
    same result keys as ``oracle_bwd.gdn2_backward`` (dq, dk, dv,
    d_log_decay, d_erase, d_write -- None when tied -- and d_state0); d_o or
    d_state None means zeros.  Gate gradients are shaped like their gates.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, dk = k.shape
    dv = v.shape[3]
    la, b, w, s0 = _f64(log_decay), _f64(erase), _f64(write), _f64(S0)
    kind = lambda g: 1 if g.shape == (B, T, H, dk) else 0
    do, ds = _f64(d_o), _f64(d_state)
    out = dict(dq=np.zeros((B, T, H, dk)), dk=np.zeros((B, T, H, dk)), dv=np.zeros((B, T, H, dv)),
               d_log_decay=np.zeros(la.shape), d_erase=np.zeros(b.shape),
               d_write=None if w is None else np.zeros(w.shape),
               d_state0=np.zeros((B, H, dk, dv)))
    nthreads = threads or available_cores()
    rc = _load().gdn2_oracle_bwd(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(la), kind(la), _ptr(b), kind(b), _ptr(w),
                                 kind(w) if w is not None else 0, _ptr(s0), float(q_scale),
                                 _ptr(do), _ptr(ds), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                 _ptr(out["d_log_decay"]), _ptr(out["d_erase"]), _ptr(out["d_write"]),
                                 _ptr(out["d_state0"]), 0, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"gradient oracle failed with code {rc}")
    return out


def prepare_inputs(q, k, x_decay, x_erase, x_write=None, qk_l2norm=True):
    """The input preparation that precedes the mixer, in fp64: the decay gate
    a = exp(-softplus(x_a)) in (0, 1) (log a = -log(1 + e^x_a)), the erase
    and write gates b = sigmoid(x_b), w = sigmoid(x_w) in (0, 1), and q, k
    divided by their L2 norm over the key channels of each token-head (a
    zero vector stays zero).  Returns (q, k, log_decay, erase, write)."""
    def l2(x):
        x = np.asarray(x, dtype=np.float64)
        n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        return np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0)

    sig = lambda x: None if x is None else 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))
    la = -np.logaddexp(0.0, np.asarray(x_decay, dtype=np.float64))
    if qk_l2norm:
        q, k = l2(q), l2(k)
    return q, k, la, sig(x_erase), sig(x_write)


def gdn2_forward_raw(q, k, v, x_decay, x_erase, x_write=None, S0=None, q_scale=1.0, qk_l2norm=True,
                     threads: int | None = None, value_write=False):
    """``gdn2_forward`` on raw inputs: gate logits and (with qk_l2norm)
    unnormalised q, k, prepared by ``prepare_inputs`` first."""
    q, k, la, b, w = prepare_inputs(q, k, x_decay, x_erase, x_write, qk_l2norm)
    return gdn2_forward(q, k, v, la, b, w, S0, q_scale=q_scale, threads=threads, value_write=value_write)


def gdn2_step(q, k, v, log_decay, erase, write, state):
    """One recurrent step for N sequences: inputs [N,H,d], gates [N,H,dk] or
    [N,H]; state [N,H,dk,dv].  Returns (o [N,H,dv], new state)."""
    add_t = lambda x: None if x is None else np.asarray(x)[:, None]
    o, S = gdn2_forward(add_t(q), add_t(k), add_t(v), add_t(log_decay),
                        add_t(erase), add_t(write), state)
    return o[:, 0], S


def max_threads() -> int:
    return int(_load().gdn2_oracle_max_threads())
