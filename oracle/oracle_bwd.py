"""TEST INFRASTRUCTURE ONLY -- gradients of the GDN-2 recurrence, fp64 on the CPU.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module; the GPU library never imports or calls it, and it
imports nothing from the GPU package.

The forward here is the token recurrence itself, written once more in plain
PyTorch float64 so that autograd can differentiate it (the C oracle beside
this file computes the same values without a tape).  Per (batch, head) chain,
with state S (dk x dv, key-by-value) and for each token t:

    Sbar = Diag(exp(la_t)) S                 decay first
    m    = Sbar^T k_t                        read the decayed state along the key
    S    = Sbar - (b_t*k_t) m^T + (w_t*k_t) v_t^T   erase with b, write with w
    o_t  = S^T (q_scale q_t)                 read the updated state

("Gated DeltaNet-2" blog summary, "Core Mechanism"; "Gated DeltaNet" page,
"Decay first, then compute the write error"; course slides, "Worked case --
full trace").  The value-write form (gist.science summary, "Methodologie",
1. "Gated Delta-regel-2") reads along b_t*k_t, erases and writes along k_t and
writes the values w_t*v_t (w per value channel):

    m    = Sbar^T (b_t*k_t)
    S    = Sbar - k_t m^T + k_t (w_t*v_t)^T

With raw inputs the preparation that precedes the mixer comes first:
log a = -softplus(x_a), b = sigmoid(x_b), w = sigmoid(x_w), and q, k divided
by their L2 norm over the key channels (a zero vector stays zero, gradient
zero there).  The gradients of a loss L with respect to every input are the
reverse-mode derivative of exactly these steps, taken by torch.autograd; no
step of the chunked form is used.  The pins in tests/test_oracle_bwd.py tie
them to central finite differences of this forward and to closed forms.
"""
from __future__ import annotations

import numpy as np
import torch


def _t(x, grad):
    if x is None:
        return None
    t = torch.as_tensor(np.asarray(x, dtype=np.float64)).clone()
    t.requires_grad_(grad)
    return t


def _per_channel(g, dk):
    """A gate [B,H] (per token-head) or [B,H,dk] (per key channel) at one
    token, as [B,H,dk]."""
    return g.unsqueeze(-1).expand(*g.shape, dk) if g.dim() == 2 else g


def recurrence(q, k, v, la, b, w, S0, q_scale=1.0, value_write=False):
    """The token recurrence on torch float64 tensors (differentiable).

    q, k [B,T,H,dk]; v [B,T,H,dv]; la, b, w [B,T,H,dk] or [B,T,H]; w None
    ties the write gate to b; S0 [B,H,dk,dv] or None (zeros).  With
    ``value_write`` the write gate is [B,T,H,dv] or [B,T,H] and the update
    is the value-write form.  Returns (o [B,T,H,dv], S_T [B,H,dk,dv]).
    """
    B, T, H, dk = k.shape
    dv = v.shape[3]
    S = S0 if S0 is not None else torch.zeros(B, H, dk, dv, dtype=torch.float64)
    outs = []
    for t in range(T):
        a = torch.exp(_per_channel(la[:, t], dk))
        bt = _per_channel(b[:, t], dk)
        kt, vt, qt = k[:, t], v[:, t], q[:, t]
        Sbar = a.unsqueeze(-1) * S
        if value_write:
            wv = _per_channel(w[:, t], dv)
            m = (Sbar * (bt * kt).unsqueeze(-1)).sum(-2)           # Sbar^T (b k)  [B,H,dv]
            S = Sbar - kt.unsqueeze(-1) * m.unsqueeze(-2) + kt.unsqueeze(-1) * (wv * vt).unsqueeze(-2)
        else:
            wt = bt if w is None else _per_channel(w[:, t], dk)
            m = (Sbar * kt.unsqueeze(-1)).sum(-2)                   # Sbar^T k   [B,H,dv]
            S = Sbar - (bt * kt).unsqueeze(-1) * m.unsqueeze(-2) + (wt * kt).unsqueeze(-1) * vt.unsqueeze(-2)
        outs.append((S * (q_scale * qt).unsqueeze(-1)).sum(-2))     # S^T (s q)  [B,H,dv]
    return torch.stack(outs, 1), S


def prepare(q, k, x_a, x_b, x_w, qk_l2norm=True):
    """The input preparation on torch float64 tensors (differentiable):
    (q, k, log a, b, w) from raw q, k and the gate logits."""
    def l2(x):
        n = torch.sqrt((x * x).sum(-1, keepdim=True))
        return torch.where(n > 0, x / torch.where(n > 0, n, torch.ones_like(n)), torch.zeros_like(x))

    la = -torch.logaddexp(torch.zeros_like(x_a), x_a)
    b = torch.sigmoid(x_b)
    w = None if x_w is None else torch.sigmoid(x_w)
    if qk_l2norm:
        q, k = l2(q), l2(k)
    return q, k, la, b, w


def gdn2_backward(q, k, v, log_decay, erase, write=None, S0=None, d_o=None, d_state=None,
                  q_scale=1.0, value_write=False, raw=False, qk_l2norm=True):
    """Gradients of L = <d_o, o> + <d_state, S_T> with respect to every input.

    Inputs as for the C oracle's ``gdn2_forward`` (numpy arrays); d_o
    [B,T,H,dv] (None: zeros), d_state [B,H,dk,dv] (None: zeros).  With
    ``raw`` the three gate arguments are logits and q, k are prepared
    (normalised when ``qk_l2norm``) first, and the gradients are those of
    the raw inputs.  Returns a dict of float64 arrays: dq, dk, dv,
    d_log_decay, d_erase, d_write (None when tied), d_state0 (the gradient
    with respect to S0, zeros-state included), plus the forward's o and S_T.
    """
    tq, tk, tv = _t(q, True), _t(k, True), _t(v, True)
    tla, tb = _t(log_decay, True), _t(erase, True)
    tw = _t(write, True) if write is not None else None
    B, T, H, dk = tk.shape
    dv = tv.shape[3]
    tS0 = _t(S0, True) if S0 is not None else torch.zeros(B, H, dk, dv, dtype=torch.float64,
                                                         requires_grad=True)
    if raw:
        pq, pk, pla, pb, pw = prepare(tq, tk, tla, tb, tw, qk_l2norm)
        o, S_T = recurrence(pq, pk, tv, pla, pb, pw, tS0, q_scale, value_write)
    else:
        o, S_T = recurrence(tq, tk, tv, tla, tb, tw, tS0, q_scale, value_write)
    loss = torch.zeros((), dtype=torch.float64)
    if d_o is not None:
        loss = loss + (o * torch.as_tensor(np.asarray(d_o, dtype=np.float64))).sum()
    if d_state is not None:
        loss = loss + (S_T * torch.as_tensor(np.asarray(d_state, dtype=np.float64))).sum()
    wrt = [tq, tk, tv, tla, tb, tS0] + ([tw] if tw is not None else [])
    if loss.requires_grad:
        grads = torch.autograd.grad(loss, wrt, allow_unused=True)
    else:
        grads = [None] * len(wrt)
    g = [np.zeros(x.shape) if gi is None else gi.detach().numpy() for x, gi in zip(wrt, grads)]
    out = dict(dq=g[0], dk=g[1], dv=g[2], d_log_decay=g[3], d_erase=g[4], d_state0=g[5],
               d_write=g[6] if tw is not None else None)
    out["o"] = o.detach().numpy()
    out["S_T"] = S_T.detach().numpy()
    return out
