"""Chunk-form gated delta rule in fp64 numpy -- TEST INFRASTRUCTURE ONLY.

This is the chunkwise algorithm the GPU path implements, written as plainly
as possible so that each intermediate can be compared with the GPU's:

  step a1  gamma: chunk-local inclusive cumsum of the log gates, in log2 units
  step a2  K+ = k * 2^gamma, K- = k * 2^-gamma, Q~ = q * 2^gamma,
           phi = 2^gamma_last, Kbar = k * 2^(gamma_last - gamma)
  step a3  A = diag(beta) StrictLower(K+ K-^T);  T = (I + A)^-1;
           W = T diag(beta) K+;  U = T diag(beta) V
  step a4  per chunk, in order: h_c = S;  Vnew = U - W S;
           S <- Diag(phi) S + Kbar^T Vnew
  step a5  O = Q~ h_c + Tril_incl(Q~ K-^T) Vnew

Orientation: here the state is the transpose of the pages' S, i.e. a
[Dk, Dv] matrix (the pages make the same choice for their kernels).

Sources:
  [KDA] "TileLang 实战：KDA 从零到一–Kimi Delta Attention":
        section 0 (gamma_i = sum_{s<=i} g_s, reset per chunk), section 1.2
        (separable exponent e^{gamma_c - gamma_i} = e^{gamma_c} e^{-gamma_i},
        M = K+ K-^T), section 3.2 (reference B: the UT system, the pseudo
        value U - W S, the output and the state update), section 3.3 item 3
        (beta applied after the triangular solve; two valid pairings).
  [SD]  "TileLang 实战：KDA 从零到一--标量衰减": section 1.2 (the three
        places the decay enters a chunk: intra-chunk ratio, write-to-chunk-end,
        read of the entry state) and section 2.3 (log domain + exp2 with
        log2(e)).
  [DPLR] "RNN的复兴04:线性注意力并行计算DPLR": section 5.3.4 (R = phi * F:
        the state-update factor is the far factor scaled by the chunk-end
        decay) and section 5.3.5 (the standard KDA/GDN chunk form and the
        four-step algorithm table).
  [EVO] "07 · linear 路线（二）：衰减机制的演进" section 3.5: the local cumsum
        restarts every chunk.

The scalar-gate kinds (gdn, decay_la) use the same formulas with gamma
broadcast over the key channels (for a scalar gate K+ K-^T equals
(K K^T) * Gamma with Gamma_ci = 2^(gamma_c - gamma_i), [SD] section 2.2).
decay_la has no delta term: Vnew = V and there is no UT transform ([SD] 1.2).

A ragged last chunk (T not a multiple of C) is simply a shorter chunk.
Library primitives used as steps: numpy matmul, numpy.cumsum, numpy.linalg.inv.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

LOG2E = 1.0 / np.log(2.0)


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def chunk_bounds(T: int, C: int) -> List[tuple]:
    return [(s, min(s + C, T)) for s in range(0, T, C)]


def chunk_log2_cumsum(g, C: int) -> np.ndarray:
    """Step a1.  g: [B,T,H,D] or [B,T,H] natural-log gates.  Returns the
    chunk-local inclusive prefix sum along T, converted to log2 units
    ([KDA] section 0; [SD] section 2.3 for the base-2 form)."""
    g = _f64(g)
    out = np.empty_like(g)
    T = g.shape[1]
    for s, e in chunk_bounds(T, C):
        out[:, s:e] = np.cumsum(g[:, s:e], axis=1) * LOG2E
    return out


def separable_prep(q, k, gamma, C: int) -> Dict[str, np.ndarray]:
    """Step a2.  q, k [B,T,H,Dk]; gamma from chunk_log2_cumsum, either
    [B,T,H,Dk] (KDA) or [B,T,H] (scalar gates, broadcast over channels).

    Returns Kp = k 2^gamma, Km = k 2^-gamma, Qp = q 2^gamma, and per chunk
    phi = 2^gamma_last [B,NT,H,Dk] and Kbar = k 2^(gamma_last - gamma)."""
    q, k, gamma = _f64(q), _f64(k), _f64(gamma)
    if gamma.ndim == 3:
        gamma = np.broadcast_to(gamma[..., None], k.shape)
    B, T, H, Dk = k.shape
    E = np.exp2(gamma)
    Ei = np.exp2(-gamma)
    bounds = chunk_bounds(T, C)
    phi = np.empty((B, len(bounds), H, Dk))
    Kbar = np.empty_like(k)
    for c, (s, e) in enumerate(bounds):
        last = gamma[:, e - 1]                      # [B,H,Dk]
        phi[:, c] = np.exp2(last)
        Kbar[:, s:e] = k[:, s:e] * np.exp2(last[:, None] - gamma[:, s:e])
    return {"Kp": k * E, "Km": k * Ei, "Qp": q * E, "phi": phi, "Kbar": Kbar}


def ut_solve(Kp: np.ndarray, Km: np.ndarray, V: np.ndarray, beta: np.ndarray):
    """Step a3 for one chunk of one head.  Kp, Km [n,Dk]; V [n,Dv]; beta [n].

    Row-beta pairing: A[c,i] = beta_c (K+ K-^T)[c,i] for i < c, T = (I+A)^-1,
    W = T diag(beta) K+, U = T diag(beta) V.  ([KDA] 3.2-3.3 lists this and
    the column-beta pairing as the two equivalent choices.)"""
    n = Kp.shape[0]
    M = np.tril(Kp @ Km.T, -1)
    A = beta[:, None] * M
    Tm = np.linalg.inv(np.eye(n) + A)
    W = Tm @ (beta[:, None] * Kp)
    U = Tm @ (beta[:, None] * V)
    return A, Tm, W, U


@dataclass
class ChunkResult:
    o: np.ndarray                      # [B,T,H,Dv]
    hT: np.ndarray                     # [B,H,Dk,Dv]  (transpose of the pages' S)
    gamma: np.ndarray                  # step a1 output
    prep: Dict[str, np.ndarray]        # step a2 outputs
    A: Optional[np.ndarray] = None     # [B,T,H,C] row blocks of A (delta kinds)
    Tinv: Optional[np.ndarray] = None  # [B,T,H,C] row blocks of T
    W: Optional[np.ndarray] = None     # [B,T,H,Dk]
    U: Optional[np.ndarray] = None     # [B,T,H,Dv]
    Vnew: Optional[np.ndarray] = None  # [B,T,H,Dv]
    Aqk: Optional[np.ndarray] = None   # [B,T,H,C]
    h: Optional[np.ndarray] = None     # [B,NT,H,Dk,Dv] entry state of each chunk
    extra: dict = field(default_factory=dict)


def chunk_forward(kind: str, q, k, v, g, beta=None, h0=None, C: int = 64,
                  ut=None) -> ChunkResult:
    """Full chunk-form forward.  kind in {"kda", "gdn", "decay_la"}.

    h0 / hT are in the kernel orientation [B,H,Dk,Dv].  ``ut`` (default
    ut_solve) computes step a3 for one chunk; tests swap it to check that a
    planted pairing mistake is caught."""
    ut = ut or ut_solve
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    beta, h0 = _f64(beta), _f64(h0)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    delta = kind in ("kda", "gdn")
    gamma = chunk_log2_cumsum(g, C)
    prep = separable_prep(q, k, gamma, C)
    Kp, Km, Qp, phi, Kbar = prep["Kp"], prep["Km"], prep["Qp"], prep["phi"], prep["Kbar"]
    bounds = chunk_bounds(T, C)
    NT = len(bounds)
    o = np.zeros((B, T, H, Dv))
    hT = np.zeros((B, H, Dk, Dv))
    A_all = np.zeros((B, T, H, C)) if delta else None
    T_all = np.zeros((B, T, H, C)) if delta else None
    W_all = np.zeros((B, T, H, Dk)) if delta else None
    U_all = np.zeros((B, T, H, Dv)) if delta else None
    Vn_all = np.zeros((B, T, H, Dv))
    Aqk_all = np.zeros((B, T, H, C))
    h_all = np.zeros((B, NT, H, Dk, Dv))
    for b in range(B):
        for hh in range(H):
            S = h0[b, hh].copy() if h0 is not None else np.zeros((Dk, Dv))
            for c, (s, e) in enumerate(bounds):
                n = e - s
                kp, km, qp = Kp[b, s:e, hh], Km[b, s:e, hh], Qp[b, s:e, hh]
                V = v[b, s:e, hh]
                h_all[b, c, hh] = S
                if delta:
                    A, Tm, W, U = ut(kp, km, V, beta[b, s:e, hh])
                    Vnew = U - W @ S
                    A_all[b, s:e, hh, :n] = A
                    T_all[b, s:e, hh, :n] = Tm
                    W_all[b, s:e, hh] = W
                    U_all[b, s:e, hh] = U
                else:
                    Vnew = V
                Aqk = np.tril(qp @ km.T)
                o[b, s:e, hh] = qp @ S + Aqk @ Vnew
                S = phi[b, c, hh][:, None] * S + Kbar[b, s:e, hh].T @ Vnew
                Vn_all[b, s:e, hh] = Vnew
                Aqk_all[b, s:e, hh, :n] = Aqk
            hT[b, hh] = S
    return ChunkResult(o=o, hT=hT, gamma=gamma, prep=prep, A=A_all, Tinv=T_all,
                       W=W_all, U=U_all, Vnew=Vn_all, Aqk=Aqk_all, h=h_all)


@dataclass
class SegmentResult:
    o: np.ndarray          # [B,T,H,Dv]
    hT: np.ndarray         # [B,H,Dk,Dv]
    o_local: np.ndarray    # [B,T,H,Dv]  output of each segment from a zero entry state
    q_eff: np.ndarray      # [B,T,H,Dk]  o = o_local + q_eff S_in(segment)
    M: np.ndarray          # [B,H,NS,Dk,Dk] transition of each segment
    N: np.ndarray          # [B,H,NS,Dk,Dv] exit state of each segment from a zero entry state
    S_in: np.ndarray       # [B,H,NS+1,Dk,Dv] entry state of each segment (last = hT)


def segment_forward(kind: str, q, k, v, g, beta=None, h0=None, C: int = 64, L: int = 2) -> SegmentResult:
    """The chunk form evaluated segment-parallel: the chunks of a sequence are
    grouped into segments of L chunks, and every segment is run from the
    augmented entry state X = [I | 0] ([Dk, Dk+Dv]).  Its first Dk columns
    carry the segment's transition P (the product of the per-token maps
    S -> (I - beta k k^T) Diag(a) S, kernel orientation), the other Dv the
    state reached from a zero entry state.  Per chunk, with U_bar = [0 | U]:
        Y = U_bar - W X,   Z = Q~ X + Aqk Y,   X <- Diag(phi) X + Kbar^T Y
    (decay_la: Y = [0 | V]).  Z's first Dk columns are the chunk's
    effective queries q_eff, the rest its output from the zero entry state.
    A segment ends with X = [M | N]; the entry states follow by
    S_in[0] = h0, S_in[r+1] = M_r S_in[r] + N_r, and o = o_local +
    q_eff S_in[segment].

    This is the entry-state hand-off of sequence-split (context-parallel)
    evaluation on [GDN] "前向计算的矩阵分解" (the chunked forward's pre-process
    that computes each split's initial state), with the segment transition
    written as the product of the per-token transition matrices, whose WY
    form is [DPLR] section 2 (D - W^T Y)."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    beta, h0 = _f64(beta), _f64(h0)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    delta = kind in ("kda", "gdn")
    gamma = chunk_log2_cumsum(g, C)
    prep = separable_prep(q, k, gamma, C)
    Kp, Km, Qp, phi, Kbar = prep["Kp"], prep["Km"], prep["Qp"], prep["phi"], prep["Kbar"]
    bounds = chunk_bounds(T, C)
    NT = len(bounds)
    NS = max(1, -(-NT // L))
    o_loc = np.zeros((B, T, H, Dv))
    q_eff = np.zeros((B, T, H, Dk))
    M = np.zeros((B, H, NS, Dk, Dk))
    N = np.zeros((B, H, NS, Dk, Dv))
    S_in = np.zeros((B, H, NS + 1, Dk, Dv))
    o = np.zeros((B, T, H, Dv))
    for b in range(B):
        for hh in range(H):
            for r in range(NS):
                X = np.concatenate([np.eye(Dk), np.zeros((Dk, Dv))], axis=1)
                for c in range(r * L, min(NT, (r + 1) * L)):
                    s, e = bounds[c]
                    kp, km, qp = Kp[b, s:e, hh], Km[b, s:e, hh], Qp[b, s:e, hh]
                    if delta:
                        _, _, W, U = ut_solve(kp, km, v[b, s:e, hh], beta[b, s:e, hh])
                        Y = np.concatenate([np.zeros((e - s, Dk)), U], axis=1) - W @ X
                    else:
                        Y = np.concatenate([np.zeros((e - s, Dk)), v[b, s:e, hh]], axis=1)
                    Z = qp @ X + np.tril(qp @ km.T) @ Y
                    q_eff[b, s:e, hh] = Z[:, :Dk]
                    o_loc[b, s:e, hh] = Z[:, Dk:]
                    X = phi[b, c, hh][:, None] * X + Kbar[b, s:e, hh].T @ Y
                M[b, hh, r], N[b, hh, r] = X[:, :Dk], X[:, Dk:]
            S_in[b, hh, 0] = h0[b, hh] if h0 is not None else 0.0
            for r in range(NS):
                S_in[b, hh, r + 1] = M[b, hh, r] @ S_in[b, hh, r] + N[b, hh, r]
            for c, (s, e) in enumerate(bounds):
                o[b, s:e, hh] = o_loc[b, s:e, hh] + q_eff[b, s:e, hh] @ S_in[b, hh, c // L]
    return SegmentResult(o=o, hT=S_in[:, :, NS].copy(), o_local=o_loc, q_eff=q_eff, M=M, N=N, S_in=S_in)
