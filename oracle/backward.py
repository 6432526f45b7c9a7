"""Backward pass of the gated delta rule, fp64 numpy -- TEST INFRASTRUCTURE ONLY.

The gradients of the token recurrence (the definition the forward oracle in
recurrence.c computes) with respect to every input, written out as the
reverse sweep over tokens.  The forward, in the pages' orientation (S in
R^{dv x dk}; page "TileLang 实战：KDA 从零到一–Kimi Delta Attention", opening
equation and section 3.1; page "Gated DeltaNet", section "DeltaNet 与 Gated
Delta Rule"):

    Sbar = S_{t-1} Diag(a_t)          a_t = exp(g_t) per key channel (kda) or
                                      one scalar per token and head
    u    = Sbar k_t                   the value the state holds at key k_t
    r    = beta_t (v_t - u)           (decay_la: r = v_t, no delta term)
    S_t  = Sbar + r k_t^T
    o_t  = S_t q_t

Reverse sweep, with the state adjoint dS (starts at dhT or zero):

    dS  += do_t q_t^T;        dq_t = S_t^T do_t
    dr   = dS k_t;            dk_t = dS^T r
    delta kinds:  dv_t = beta_t dr;  du = -beta_t dr;  dbeta_t = dr . (v_t - u)
                  dS += du k_t^T;    dk_t += Sbar^T du
    decay_la:     dv_t = dr
    da   = column sums of dS * S_{t-1};   dg_t = a_t * da  (summed over the
                                          channels for a scalar gate)
    dS   = dS Diag(a_t)                    (the adjoint of S_{t-1})

and dh0 = dS after the first token.  This is the derivative of the forward
with nothing reordered; it is pinned by central finite differences through
the forward oracle and by the closed form of scalar-decay linear attention
(tests/test_oracle_pins.py).
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _f64(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def recurrence_backward(kind: str, q, k, v, g, beta=None, h0=None, do=None, dhT=None):
    """Gradients of the token recurrence.

    kind: "kda" | "gdn" | "decay_la".
    q, k: [B,T,H,Dk]; v: [B,T,H,Dv]; g: [B,T,H,Dk] (kda) or [B,T,H];
    beta: [B,T,H] (None for decay_la); h0: [B,H,Dv,Dk] (pages' orientation)
    or None; do: [B,T,H,Dv] (None = zero); dhT: [B,H,Dv,Dk] or None.
    Returns dict with dq, dk, dv, dg (shape of g), dbeta (None for
    decay_la), dh0 [B,H,Dv,Dk], and the forward's o and hT.
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    beta, h0, do, dhT = _f64(beta), _f64(h0), _f64(do), _f64(dhT)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    delta = kind != "decay_la"
    perch = kind == "kda"
    if do is None:
        do = np.zeros((B, T, H, Dv))
    out = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dg", g))}
    out["dbeta"] = np.zeros_like(beta) if delta else None
    out["dh0"] = np.zeros((B, H, Dv, Dk))
    out["o"] = np.zeros((B, T, H, Dv))
    out["hT"] = np.zeros((B, H, Dv, Dk))
    for b in range(B):
        for h in range(H):
            # forward, keeping every state S_0 .. S_T
            S = np.zeros((T + 1, Dv, Dk))
            if h0 is not None:
                S[0] = h0[b, h]
            for t in range(T):
                a = np.exp(g[b, t, h])                       # [Dk] or scalar
                Sbar = S[t] * a
                kt = k[b, t, h]
                if delta:
                    u = Sbar @ kt
                    r = beta[b, t, h] * (v[b, t, h] - u)
                else:
                    r = v[b, t, h]
                S[t + 1] = Sbar + np.outer(r, kt)
                out["o"][b, t, h] = S[t + 1] @ q[b, t, h]
            out["hT"][b, h] = S[T]
            # reverse sweep
            dS = np.zeros((Dv, Dk)) if dhT is None else dhT[b, h].copy()
            for t in range(T - 1, -1, -1):
                a = np.exp(g[b, t, h])
                Sbar = S[t] * a
                kt, qt, dot = k[b, t, h], q[b, t, h], do[b, t, h]
                dS += np.outer(dot, qt)
                out["dq"][b, t, h] = S[t + 1].T @ dot
                if delta:
                    u = Sbar @ kt
                    r = beta[b, t, h] * (v[b, t, h] - u)
                else:
                    r = v[b, t, h]
                dr = dS @ kt
                dkt = dS.T @ r
                if delta:
                    out["dv"][b, t, h] = beta[b, t, h] * dr
                    du = -beta[b, t, h] * dr
                    out["dbeta"][b, t, h] = dr @ (v[b, t, h] - u)
                    dS = dS + np.outer(du, kt)
                    dkt = dkt + Sbar.T @ du
                else:
                    out["dv"][b, t, h] = dr
                out["dk"][b, t, h] = dkt
                da = np.sum(dS * S[t], axis=0)               # [Dk]
                out["dg"][b, t, h] = a * da if perch else a * np.sum(da)
                dS = dS * a
            out["dh0"][b, h] = dS
    return out
