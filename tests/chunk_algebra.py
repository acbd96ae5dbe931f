"""fp64 numpy statement of the chunkwise-parallel (WY/UT) form -- test helper.

Not the oracle and not the product: it writes down, in plain numpy, the
chunk algebra that the GPU kernels implement, so that a CPU test can show it
equals the token recurrence (the oracle) before any kernel relies on it.  The
gist.science summary ("Technische Samenvatting", section 3) names the
ingredients: the cumulative per-channel decay is absorbed into the erase and
write factors, and a unit-lower-triangular solve (I+T)^-1 gives the auxiliary
matrices.  The form below is derived for the key-axis erase/write gates.

Within a chunk of C tokens entering with state S (dk x dv), with g_r the
inclusive cumulative log-decay inside the chunk (per key channel), e = b*k,
u = w*k:

    A[r,s] = sum_c k_r[c] e_s[c] exp(g_r[c]-g_s[c])   (r > s),  Bm: u in place of e
    R[r,s] = sum_c q_r[c] e_s[c] exp(g_r[c]-g_s[c])   (r >= s), P:  u in place of e
    Kbar = k * exp(g),  Qbar = q * exp(g)
    M = (I + A)^-1 (Kbar S + Bm V)          rows m_r = (decayed state before r)^T k_r
    O = Qbar S + P V - R M
    S <- exp(g_C) * S + Utilde^T V - Etilde^T M,   Utilde_s = u_s exp(g_C - g_s), same for E

``hook(name, x)`` may replace any named intermediate (used to emulate the
rounding of operands); by default it is the identity.
"""
from __future__ import annotations

import numpy as np


def _ident(name, x):
    return x


def chunk_forward(q, k, v, log_decay, erase, write=None, S0=None, chunk=16,
                  q_scale=1.0, hook=_ident):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, H, dk = k.shape
    dv = v.shape[-1]

    def per_key(g):
        g = np.asarray(g, dtype=np.float64)
        return g if g.ndim == 4 else np.repeat(g[..., None], dk, axis=-1)

    la = per_key(log_decay)
    b = per_key(erase)
    w = b if write is None else per_key(write)
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((B, H, dk, dv))
    for bi in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[bi, h], dtype=np.float64)
            for t0 in range(0, T, chunk):
                t1 = min(T, t0 + chunk)
                K = k[bi, t0:t1, h]
                Q = q_scale * q[bi, t0:t1, h]
                V = v[bi, t0:t1, h]
                g = np.cumsum(la[bi, t0:t1, h], axis=0)
                E = b[bi, t0:t1, h] * K
                U = w[bi, t0:t1, h] * K
                C = t1 - t0
                D = np.exp(g[:, None, :] - g[None, :, :])  # [r,s,c]; used only for r >= s
                low = np.tril(np.ones((C, C)), -1)
                incl = np.tril(np.ones((C, C)), 0)
                with np.errstate(over="ignore", invalid="ignore"):
                    A = low * np.nan_to_num(np.einsum("rc,sc,rsc->rs", K, E, D))
                    Bm = low * np.nan_to_num(np.einsum("rc,sc,rsc->rs", K, U, D))
                    R = incl * np.nan_to_num(np.einsum("rc,sc,rsc->rs", Q, E, D))
                    P = incl * np.nan_to_num(np.einsum("rc,sc,rsc->rs", Q, U, D))
                A, Bm, R, P = (hook(n, x) for n, x in (("A", A), ("B", Bm), ("R", R), ("P", P)))
                Tinv = hook("T", np.linalg.inv(np.eye(C) + A))
                Kbar = hook("Kbar", K * np.exp(g))
                Qbar = hook("Qbar", Q * np.exp(g))
                Sx = hook("S", S)
                X = hook("X", Kbar @ Sx + Bm @ V)
                M = hook("M", Tinv @ X)
                O = Qbar @ Sx + P @ V - R @ M
                o[bi, t0:t1, h] = hook("O", O)
                Et = hook("Etil", E * np.exp(g[-1] - g))
                Ut = hook("Util", U * np.exp(g[-1] - g))
                S = np.exp(g[-1])[:, None] * S + Ut.T @ V - Et.T @ M
            S_T[bi, h] = S
    return o, S_T
