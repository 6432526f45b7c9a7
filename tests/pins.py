"""Pins of the CPU oracle: checks against what the pages and the mathematics
fix, independent of the oracle's own code.

Each pin takes ``rec`` -- a callable with the signature of
``oracle.recurrence`` -- so the same pins can be run against deliberately
broken copies of the oracle (see test_oracle_pins.py) to show that they
catch plausible mistakes.  Every pin raises AssertionError on failure.

Page keys: [SD] "TileLang 实战：KDA 从零到一--标量衰减"; [KDA] "TileLang
实战：KDA 从零到一–Kimi Delta Attention"; [GDN] "Gated DeltaNet";
[DPLR] "RNN的复兴04:线性注意力并行计算DPLR";
[EVO] "07 · linear 路线（二）：衰减机制的演进".
"""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rel(a, b):
    """max |a-b| / max |b| (the infinity-norm relative error)."""
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def rand_case(kind, B=2, T=12, H=2, Dk=4, Dv=4, seed=0, gate=(0.9, 0.999),
              beta=(0.1, 0.9), h0_std=0.0, l2=True):
    """fp64 random inputs in the pages' test recipe ([KDA] 3.4: a ~ U(0.9,
    0.999)^dk, beta ~ U(0.1, 0.9), L2-normalised q and k)."""
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, H, Dk))
    k = r.standard_normal((B, T, H, Dk))
    if l2:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, T, H, Dv))
    gshape = (B, T, H, Dk) if kind == "kda" else (B, T, H)
    g = np.log(r.uniform(gate[0], gate[1], gshape))
    bt = r.uniform(beta[0], beta[1], (B, T, H))
    h0 = r.standard_normal((B, H, Dv, Dk)) * h0_std if h0_std > 0 else None
    return q, k, v, g, bt, h0


# --------------------------------------------------------------------------
# (a) scalar decay without delta == parallel retention / SSD dual form
# --------------------------------------------------------------------------
def pin_retention_parallel(rec):
    """[EVO] section 1, Eq. 5: with a constant per-head decay gamma_h the
    recurrence equals (Q K^T .* D) V, D_nm = gamma^(n-m) for n >= m, else 0
    (D evaluated only where n >= m, [SD] 2.2).  gamma_h = 1 - 2^(-5-h) is the
    multi-scale schedule of the same section."""
    B, T, H, D = 1, 96, 4, 8
    r = np.random.default_rng(1)
    q, k, v = (r.standard_normal((B, T, H, D)) for _ in range(3))
    gam = 1.0 - 2.0 ** (-5.0 - np.arange(H))
    g = np.broadcast_to(np.log(gam)[None, None, :], (B, T, H)).copy()
    o, _ = rec("decay_la", q, k, v, g)
    n = np.arange(T)
    for h in range(H):
        Dm = np.zeros((T, T))
        for i in range(T):
            Dm[i, : i + 1] = gam[h] ** (i - n[: i + 1])
        ref = ((q[0, :, h] @ k[0, :, h].T) * Dm) @ v[0, :, h]
        assert rel(o[0, :, h], ref) < 1e-12, "retention parallel form"


def pin_ssd_dual(rec):
    """[EVO] sections 3.2 and 3.5: with a per-token scalar decay the recurrence
    equals (Q K^T .* L) V with L_ij = exp(G_i - G_j) for i >= j (G the running
    sum of log gates), plus the entry-state read exp(G_i) S_0 q_i."""
    B, T, H, D = 2, 80, 2, 6
    r = np.random.default_rng(2)
    q, k, v = (r.standard_normal((B, T, H, D)) for _ in range(3))
    g = np.log(r.uniform(0.85, 0.999, (B, T, H)))
    h0 = r.standard_normal((B, H, D, D))
    o, hT = rec("decay_la", q, k, v, g, None, h0)
    for b in range(B):
        for h in range(H):
            G = np.cumsum(g[b, :, h])
            L = np.zeros((T, T))
            for i in range(T):
                L[i, : i + 1] = np.exp(G[i] - G[: i + 1])
            ref = ((q[b, :, h] @ k[b, :, h].T) * L) @ v[b, :, h]
            ref += np.exp(G)[:, None] * (q[b, :, h] @ h0[b, h].T)
            assert rel(o[b, :, h], ref) < 1e-12, "SSD dual form"
            Sref = np.exp(G[-1]) * h0[b, h] + (v[b, :, h] * np.exp(G[-1] - G)[:, None]).T @ k[b, :, h]
            assert rel(hT[b, h], Sref) < 1e-12, "SSD final state"


# --------------------------------------------------------------------------
# (b) DPLR WY representation, brute force on tiny inputs
# --------------------------------------------------------------------------
def _dplr_operands(a, k, v, bt):
    """Map one KDA chain onto the pages' DPLR form ([DPLR] section 3.1):
    S_t = S_{t-1} [Lambda_t - x_t y_t^T] + v'_t k_t^T with Lambda_t = Diag(a_t),
    x_t = beta_t (a_t * k_t), y_t = k_t, v'_t = beta_t v_t."""
    return a, bt[:, None] * a * k, k, bt[:, None] * v


def wy_factors(lam, x, y, kk, vv, t):
    """[DPLR] section 2 and 3.1 recursions up to step t (1-based):
      w_s   = D_{s-1} x_s - sum_{tau<s} (nu_tau^(s-1)^T x_s) w_tau
      u_s   = v'_s      - sum_{tau<s} (kappa_tau^(s-1)^T x_s) u_tau
      nu_tau^(s) = D_{tau+1:s} y_tau,  kappa_tau^(s) = D_{tau+1:s} k_tau.
    Returns D_t, W_t^T Y_t and U_t^T K_t."""
    n = lam.shape[1]
    logD = np.vstack([np.zeros(n), np.cumsum(np.log(lam[:t]), axis=0)])  # logD[s] = log diag D_s

    def Dr(s0, s1):  # diag of D_{s0:s1} = prod_{s0 <= s <= s1} Lambda_s (1-based, inclusive)
        return np.exp(logD[s1] - logD[s0 - 1])

    ws, us = [], []
    for s in range(1, t + 1):
        xs = x[s - 1]
        w = np.exp(logD[s - 1]) * xs
        u = vv[s - 1].copy()
        for tau in range(1, s):
            nu = Dr(tau + 1, s - 1) * y[tau - 1]
            kap = Dr(tau + 1, s - 1) * kk[tau - 1]
            w = w - (nu @ xs) * ws[tau - 1]
            u = u - (kap @ xs) * us[tau - 1]
        ws.append(w)
        us.append(u)
    Dt = np.diag(np.exp(logD[t]))
    WY = sum(np.outer(ws[tau - 1], Dr(tau + 1, t) * y[tau - 1]) for tau in range(1, t + 1))
    UK = sum(np.outer(us[tau - 1], Dr(tau + 1, t) * kk[tau - 1]) for tau in range(1, t + 1))
    return Dt, WY, UK


def pin_wy_brute_force(rec):
    """[DPLR] section 2: prod_{tau<=t} (Lambda_tau - x_tau y_tau^T) = D_t - W_t^T Y_t
    (matrices multiplied out directly), and section 3.1:
    S_t = S_0 [D_t - W_t^T Y_t] + U_t^T K_t, compared with the oracle's state
    after t tokens.  Tiny sizes, every t up to 12."""
    r = np.random.default_rng(3)
    for Dk in (2, 4):
        Dv = 3
        T = 12
        q, k, v, g, bt, h0 = rand_case("kda", B=1, T=T, H=1, Dk=Dk, Dv=Dv, seed=10 + Dk, h0_std=1.0)
        a = np.exp(g[0, :, 0])
        lam, x, y, vv = _dplr_operands(a, k[0, :, 0], v[0, :, 0], bt[0, :, 0])
        P = np.eye(Dk)
        for t in range(1, T + 1):
            P = P @ (np.diag(lam[t - 1]) - np.outer(x[t - 1], y[t - 1]))
            Dt, WY, UK = wy_factors(lam, x, y, k[0, :, 0], vv, t)
            assert rel(Dt - WY, P) < 1e-12, "WY identity"
            _, hT = rec("kda", q[:, :t], k[:, :t], v[:, :t], g[:, :t], bt[:, :t], h0)
            St = h0[0, 0] @ (Dt - WY) + UK
            assert rel(hT[0, 0], St) < 1e-12, "DPLR parallel state"
    _ = r


def pin_iplr_wy(rec):
    """[DPLR] section 1.2 (IPLR, no decay): with g = 0 the delta rule's state is
    S_t = S_0 (I - W^T Y) + U^T K with w_t = x_t - sum (y_tau^T x_t) w_tau;
    the gated rule with g = 0 is DeltaNet ([KDA] 3.4, third reduction)."""
    T, Dk, Dv = 10, 4, 3
    q, k, v, _, bt, h0 = rand_case("gdn", B=1, T=T, H=1, Dk=Dk, Dv=Dv, seed=21, h0_std=1.0)
    g = np.zeros((1, T, 1))
    kk = k[0, :, 0]
    x = bt[0, :, 0][:, None] * kk
    vv = bt[0, :, 0][:, None] * v[0, :, 0]
    ws, us = [], []
    for t in range(T):
        w = x[t] - sum((kk[tau] @ x[t]) * ws[tau] for tau in range(t)) if t else x[t].copy()
        u = vv[t] - sum((kk[tau] @ x[t]) * us[tau] for tau in range(t)) if t else vv[t].copy()
        ws.append(w)
        us.append(u)
    S = h0[0, 0] @ (np.eye(Dk) - np.array(ws).T @ kk) + np.array(us).T @ kk
    _, hT = rec("gdn", q, k, v, g, bt, h0)
    assert rel(hT[0, 0], S) < 1e-12, "IPLR WY state"


# --------------------------------------------------------------------------
# (d) reductions
# --------------------------------------------------------------------------
def pin_beta_zero_pure_decay(rec):
    """beta = 0 leaves only the decay: S_T = S_0 Diag(exp sum_t g_t) and
    o_t = S_0 (exp(sum_{s<=t} g_s) * q_t) ([KDA] 3.4, second reduction, in
    closed form), for both the per-channel and the scalar gate."""
    for kind in ("kda", "gdn"):
        q, k, v, g, _, h0 = rand_case(kind, B=1, T=20, H=2, Dk=5, Dv=3, seed=31, h0_std=1.0)
        bt = np.zeros((1, 20, 2))
        o, hT = rec(kind, q, k, v, g, bt, h0)
        G = np.cumsum(g, axis=1)
        if kind == "gdn":
            G = np.broadcast_to(G[..., None], q.shape)
        for h in range(2):
            ref_o = (q[0, :, h] * np.exp(G[0, :, h])) @ h0[0, h].T
            assert rel(o[0, :, h], ref_o) < 1e-12, "beta=0 output"
            assert rel(hT[0, h], h0[0, h] * np.exp(G[0, -1, h])[None, :]) < 1e-12, "beta=0 state"


def pin_vanilla_linear_attention(rec):
    """decay_la with g = 0 is causal linear attention ([SD] 1.0 first
    equation; 4.4 last row): O = tril(Q K^T) V + Q S_0^T."""
    B, T, H, D = 1, 40, 2, 6
    r = np.random.default_rng(41)
    q, k, v = (r.standard_normal((B, T, H, D)) for _ in range(3))
    h0 = r.standard_normal((B, H, D, D))
    o, hT = rec("decay_la", q, k, v, np.zeros((B, T, H)), None, h0)
    for h in range(H):
        ref = np.tril(q[0, :, h] @ k[0, :, h].T) @ v[0, :, h] + q[0, :, h] @ h0[0, h].T
        assert rel(o[0, :, h], ref) < 1e-12, "vanilla LA"
        assert rel(hT[0, h], h0[0, h] + v[0, :, h].T @ k[0, :, h]) < 1e-12


def pin_kda_channel_equal_is_gdn(rec):
    """[KDA] 3.4, first reduction: a per-channel gate with all channels equal
    must give exactly the scalar-gate (GDN) result."""
    q, k, v, g, bt, h0 = rand_case("gdn", B=2, T=24, H=2, Dk=6, Dv=5, seed=51, h0_std=0.5)
    gk = np.broadcast_to(g[..., None], q.shape).copy()
    o1, s1 = rec("gdn", q, k, v, g, bt, h0)
    o2, s2 = rec("kda", q, k, v, gk, bt, h0)
    assert rel(o2, o1) < 1e-13 and rel(s2, s1) < 1e-13, "KDA(channel-equal) == GDN"


def pin_per_channel_gate_position(rec):
    """Diag(a_t) sits between S_{t-1} and the Householder factor ([KDA] 3.1):
    one token from a known state, checked against the formula multiplied out
    with explicit matrices (so a gate applied on the wrong side, after the
    update, or to the wrong channel is caught)."""
    Dk, Dv = 4, 3
    r = np.random.default_rng(61)
    S0 = r.standard_normal((Dv, Dk))
    k = r.standard_normal(Dk); k /= np.linalg.norm(k)
    q = r.standard_normal(Dk)
    v = r.standard_normal(Dv)
    a = np.array([0.5, 0.7, 0.9, 0.95])
    b = 0.6
    S1 = S0 @ np.diag(a) @ (np.eye(Dk) - b * np.outer(k, k)) + b * np.outer(v, k)
    o, hT = rec("kda", q[None, None, None], k[None, None, None], v[None, None, None],
                np.log(a)[None, None, None], np.array([[[b]]]), S0[None, None])
    assert rel(hT[0, 0], S1) < 1e-14 and rel(o[0, 0, 0], S1 @ q) < 1e-14, "one KDA step"


# --------------------------------------------------------------------------
# (f) invariant of the delta update
# --------------------------------------------------------------------------
def pin_delta_replacement(rec):
    """With a_t = 1 and unit keys the update gives
    S_t k_t = (1 - beta_t) S_{t-1} k_t + beta_t v_t; for beta = 1 the old value
    along k_t is replaced by v_t ([GDN] "DeltaNet 与 Gated Delta Rule").
    Checked at every step by chaining one-token calls through h0/hT."""
    Dk, Dv, T = 5, 4, 15
    q, k, v, _, bt, h0 = rand_case("gdn", B=1, T=T, H=1, Dk=Dk, Dv=Dv, seed=71, h0_std=1.0)
    bt[0, ::3, 0] = 1.0
    g = np.zeros((1, 1, 1))
    S = h0
    for t in range(T):
        sl = slice(t, t + 1)
        _, S1 = rec("gdn", q[:, sl], k[:, sl], v[:, sl], g, bt[:, sl], S)
        kt, b = k[0, t, 0], bt[0, t, 0]
        lhs = S1[0, 0] @ kt
        rhs = (1 - b) * (S[0, 0] @ kt) + b * v[0, t, 0]
        assert rel(lhs, rhs) < 1e-12, "delta invariant"
        S = S1


def pin_resume(rec):
    """The final state is the hand-over point: running [0, T1) then [T1, T)
    from the first call's state equals one call over [0, T)."""
    for kind in ("kda", "gdn", "decay_la"):
        q, k, v, g, bt, h0 = rand_case(kind, B=2, T=30, H=2, Dk=4, Dv=3, seed=81, h0_std=0.3)
        bt_ = None if kind == "decay_la" else bt
        o, s = rec(kind, q, k, v, g, bt_, h0)
        o1, s1 = rec(kind, q[:, :11], k[:, :11], v[:, :11], g[:, :11], None if bt_ is None else bt_[:, :11], h0)
        o2, s2 = rec(kind, q[:, 11:], k[:, 11:], v[:, 11:], g[:, 11:], None if bt_ is None else bt_[:, 11:], s1)
        assert rel(np.concatenate([o1, o2], 1), o) < 1e-13 and rel(s2, s) < 1e-13, "resume"


def pin_chunk_form_equals_recurrence(rec, chunked):
    """The chunk form ([KDA] 3.2 reference B, [DPLR] 5.3.5) must equal the
    recurrence to rounding: the pages report ~1e-16 on B=2,H=2,T=12,d=4,C=4
    ([KDA] 3.4, [SD] 4.4).  Also C = 1 (every chunk one token, the strictly
    lower part vanishes) and a ragged last chunk."""
    for kind in ("kda", "gdn", "decay_la"):
        for (T, C) in ((12, 4), (12, 1), (23, 8), (40, 16)):
            q, k, v, g, bt, h0 = rand_case(kind, B=2, T=T, H=2, Dk=4, Dv=4, seed=91 + T + C, h0_std=0.5)
            bt_ = None if kind == "decay_la" else bt
            o, s = rec(kind, q, k, v, g, bt_, h0)
            res = chunked.chunk_forward(kind, q, k, v, g, bt_, np.swapaxes(h0, -1, -2), C)
            assert rel(res.o, o) < 1e-12, f"chunk form output {kind} T={T} C={C}"
            assert rel(np.swapaxes(res.hT, -1, -2), s) < 1e-12, f"chunk form state {kind} T={T} C={C}"


def _token_maps(kind, k, g, bt):
    """Per-token transition maps of one (b, h) chain in kernel orientation
    (state [Dk, Dv]): S -> (I - beta k k^T) Diag(a) S, decay_la: Diag(a) S,
    built directly from the recurrence's definition ([KDA] opening equation,
    transposed)."""
    T, Dk = k.shape
    out = []
    for t in range(T):
        a = np.exp(g[t]) * np.ones(Dk)
        F = np.diag(a)
        if kind != "decay_la":
            F = (np.eye(Dk) - bt[t] * np.outer(k[t], k[t])) @ F
        out.append(F)
    return out


def pin_segment_form(rec, chunked):
    """The segment-parallel evaluation (chunks grouped into segments, each run
    from [I | 0], entry states composed afterwards) must equal the recurrence
    to rounding, for segments of 1, several and more than all chunks and a
    ragged tail; and its pieces must be what they claim, checked against
    products of the per-token maps written out directly: each segment's
    transition M_r is the product of its tokens' maps in time order, N_r the
    recurrence from a zero state over its tokens, and the effective query of
    token t is q_t^T times the product of the maps from the segment's first
    token through t."""
    for kind in ("kda", "gdn", "decay_la"):
        for (T, C, L) in ((40, 4, 3), (23, 8, 1), (12, 4, 9), (33, 4, 2)):
            q, k, v, g, bt, h0 = rand_case(kind, B=2, T=T, H=2, Dk=4, Dv=3, seed=131 + T + L, h0_std=0.5)
            bt_ = None if kind == "decay_la" else bt
            o, s = rec(kind, q, k, v, g, bt_, h0)
            res = chunked.segment_forward(kind, q, k, v, g, bt_, np.swapaxes(h0, -1, -2), C, L)
            assert rel(res.o, o) < 1e-12, f"segment form output {kind} T={T} C={C} L={L}"
            assert rel(np.swapaxes(res.hT, -1, -2), s) < 1e-12, f"segment form state {kind} T={T} L={L}"
            b, hh = 1, 0
            maps = _token_maps(kind, k[b, :, hh], g[b, :, hh], None if bt_ is None else bt_[b, :, hh])
            for r in range(res.M.shape[2]):
                t0, t1 = r * L * C, min(T, (r + 1) * L * C)
                P = np.eye(k.shape[-1])
                for t in range(t0, t1):
                    P = maps[t] @ P
                    qe = q[b, t, hh] @ P
                    assert rel(res.q_eff[b, t, hh], qe) < 1e-12, f"effective query {kind} t={t}"
                assert rel(res.M[b, hh, r], P) < 1e-12, f"segment transition {kind} r={r}"
                _, sN = rec(kind, q[b:b + 1, t0:t1], k[b:b + 1, t0:t1], v[b:b + 1, t0:t1], g[b:b + 1, t0:t1],
                            None if bt_ is None else bt_[b:b + 1, t0:t1], None)
                assert rel(res.N[b, hh, r], sN[0, hh].T) < 1e-12, f"segment exit state {kind} r={r}"


ALL_RECURRENCE_PINS = [
    pin_retention_parallel, pin_ssd_dual, pin_wy_brute_force, pin_iplr_wy,
    pin_beta_zero_pure_decay, pin_vanilla_linear_attention,
    pin_kda_channel_equal_is_gdn, pin_per_channel_gate_position,
    pin_delta_replacement, pin_resume,
]


def read_golden(name):
    """Parse a [section]-structured text fixture into {section: ndarray}."""
    out, cur, rows = {}, None, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("["):
                if cur is not None:
                    out[cur] = np.array(rows, dtype=np.float64)
                cur, rows = line[1:-1], []
            else:
                rows.append([float(x) for x in line.split()])
    if cur is not None:
        out[cur] = np.array(rows, dtype=np.float64)
    return out


# --------------------------------------------------------------------------
# Input prologue ([GDN] sections "门控与 Head 映射" and "加载 Token 与写入系数").
# Each pin takes ``pro`` -- a module with the interface of oracle.prologue --
# so the pins can be run against broken copies of it.
# --------------------------------------------------------------------------
def pin_l2_normalize(pro):
    """x / sqrt(|x|^2 + 1e-6) per token and head: closed forms and the
    per-row invariant."""
    # [3, 4] -> [0.6, 0.8] up to the epsilon: 25 / (25 + 1e-6) of unit norm
    y = pro.l2_normalize(np.array([[[[3.0, 4.0]]]]))
    assert rel(y[0, 0, 0], np.array([0.6, 0.8])) < 1e-7
    # a row whose squares sum to exactly the epsilon: [1e-3, 0] -> [1/sqrt(2), 0]
    y = pro.l2_normalize(np.array([[[[1e-3, 0.0]]]]))
    assert abs(y[0, 0, 0, 0] - 2 ** -0.5) < 1e-12 and y[0, 0, 0, 1] == 0.0
    # the zero row stays zero
    assert np.all(pro.l2_normalize(np.zeros((1, 2, 3, 4))) == 0.0)
    # every [b, t, h, :] row separately: |y|^2 = s / (s + eps), direction kept
    r = np.random.default_rng(40)
    x = r.standard_normal((2, 5, 3, 8)) * r.uniform(0.1, 10.0, (2, 5, 3, 1))
    y = pro.l2_normalize(x)
    s = np.sum(x * x, axis=-1)
    assert rel(np.sum(y * y, axis=-1), s / (s + 1e-6)) < 1e-13
    cos = np.sum(x * y, axis=-1) / np.sqrt(s * np.sum(y * y, axis=-1))
    assert np.max(np.abs(cos - 1.0)) < 1e-13


def pin_sigmoid_softplus(pro):
    """sigmoid(ln 3) = 3/4, sigmoid(x) + sigmoid(-x) = 1; softplus(0) = ln 2,
    softplus(ln(e - 1)) = 1, softplus(x) - softplus(-x) = x, no overflow."""
    assert abs(pro.sigmoid(np.log(3.0)) - 0.75) < 1e-15
    assert abs(pro.sigmoid(-np.log(3.0)) - 0.25) < 1e-15
    assert pro.sigmoid(0.0) == 0.5
    x = np.linspace(-30, 30, 121)
    assert np.max(np.abs(pro.sigmoid(x) + pro.sigmoid(-x) - 1.0)) < 1e-15
    assert abs(pro.softplus(0.0) - np.log(2.0)) < 1e-15
    assert abs(pro.softplus(np.log(np.e - 1.0)) - 1.0) < 1e-15
    assert np.max(np.abs(pro.softplus(x) - pro.softplus(-x) - x)) < 1e-12
    assert pro.softplus(800.0) == 800.0 and 0.0 < pro.softplus(-700.0) < 1e-300


def pin_scalar_gate(pro):
    """g = -exp(A_log[h]) softplus(a + dt_bias[h]): a worked value per head,
    g < 0 everywhere, and the large-input asymptote -exp(A_log)(a + dt)."""
    A_log = np.log(np.array([2.0, 0.5, 16.0]))
    dt = np.array([0.5, -1.0, 0.0])
    # a chosen per head so that a + dt = ln(e - 1): softplus = 1, g = -exp(A_log)
    a = np.broadcast_to(np.log(np.e - 1.0) - dt, (2, 4, 3)).copy()
    g = pro.scalar_gate(a, A_log, dt)
    assert rel(g, np.broadcast_to(-np.array([2.0, 0.5, 16.0]), (2, 4, 3))) < 1e-14
    r = np.random.default_rng(41)
    a = r.standard_normal((2, 6, 3)) * 4.0
    g = pro.scalar_gate(a, A_log, dt)
    assert np.all(g < 0.0)
    big = pro.scalar_gate(np.full((1, 1, 3), 50.0), A_log, dt)
    assert rel(big[0, 0], -np.array([2.0, 0.5, 16.0]) * (50.0 + dt)) < 1e-14
    # no bias = zero bias
    assert rel(pro.scalar_gate(a, A_log), pro.scalar_gate(a, A_log, np.zeros(3))) == 0.0


def pin_prologue_order(pro):
    """The scale applies after the normalisation (|q| = scale), beta_x2
    doubles the sigmoid, and with every option off the inputs pass through."""
    r = np.random.default_rng(42)
    q, k = (r.standard_normal((1, 3, 2, 16)) * 5.0 for _ in range(2))
    g, b = r.standard_normal((1, 3, 2)), r.standard_normal((1, 3, 2))
    q2, k2, g2, b2 = pro.apply("gdn", q, k, g, b, qk_l2norm=True, scale=0.25, beta_sigmoid=True,
                               beta_x2=True)
    assert np.max(np.abs(np.linalg.norm(q2, axis=-1) - 0.25)) < 1e-8
    assert np.max(np.abs(np.linalg.norm(k2, axis=-1) - 1.0)) < 1e-8
    assert rel(b2, 2.0 / (1.0 + np.exp(-b))) < 1e-15 and np.array_equal(g2, g)
    q3, k3, g3, b3 = pro.apply("kda", q, k, g, b)
    assert all(np.array_equal(x, y) for x, y in ((q3, q), (k3, k), (g3, g), (b3, b)))


def pin_prologue_householder(pro, rec):
    """Through the recurrence: with q = k (raw, same vector), L2
    normalisation, beta = 2 sigmoid(0) = 1 and no decay, each step is the
    Householder write S k = v, so o_t = v_t up to the epsilon's deficit in
    |k|^2 ([GDN] section "DeltaNet 与 Gated Delta Rule": unit keys and beta = 1
    give a reflection that writes v at k)."""
    r = np.random.default_rng(43)
    B, T, H, D = 1, 10, 2, 8
    k = r.standard_normal((B, T, H, D)) * 3.0
    v = r.standard_normal((B, T, H, D))
    q2, k2, g2, b2 = pro.apply("gdn", k.copy(), k, np.zeros((B, T, H)), np.zeros((B, T, H)),
                               qk_l2norm=True, beta_sigmoid=True, beta_x2=True)
    o, _ = rec("gdn", q2, k2, v, g2, b2)
    assert rel(o, v) < 1e-5


ALL_PROLOGUE_PINS = [pin_l2_normalize, pin_sigmoid_softplus, pin_scalar_gate, pin_prologue_order]


# --------------------------------------------------------------------------
# Backward pass (oracle/backward.py).  Each pin takes ``bwd`` -- a callable
# with the signature of oracle.backward.recurrence_backward -- so that broken
# copies can be run through them.
# --------------------------------------------------------------------------
def _fd_case(kind, seed):
    r = np.random.default_rng(seed)
    B, T, H, Dk, Dv = 1, 6, 2, 3, 4
    q, k = r.standard_normal((B, T, H, Dk)), r.standard_normal((B, T, H, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, T, H, Dv))
    g = np.log(r.uniform(0.5, 0.99, (B, T, H, Dk) if kind == "kda" else (B, T, H)))
    bt = r.uniform(0.2, 0.9, (B, T, H)) if kind != "decay_la" else None
    h0 = r.standard_normal((B, H, Dv, Dk)) * 0.5
    do = r.standard_normal((B, T, H, Dv))
    dhT = r.standard_normal((B, H, Dv, Dk))
    return dict(q=q, k=k, v=v, g=g, beta=bt, h0=h0), do, dhT


def pin_backward_finite_differences(bwd, rec):
    """Every gradient against central differences of the loss
    L = <do, o> + <dhT, hT> evaluated by the forward oracle, on small random
    inputs of each kind (with an initial state and a final-state cotangent)."""
    eps = 1e-6
    for kind in ("kda", "gdn", "decay_la"):
        x, do, dhT = _fd_case(kind, {"kda": 60, "gdn": 61, "decay_la": 62}[kind])

        def loss(xx):
            o, hT = rec(kind, xx["q"], xx["k"], xx["v"], xx["g"], xx["beta"], xx["h0"])
            return float(np.sum(o * do) + np.sum(hT * dhT))

        grads = bwd(kind, x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], do, dhT)
        for name in ("q", "k", "v", "g", "beta", "h0"):
            if x[name] is None:
                continue
            gnum = np.zeros_like(x[name])
            it = np.nditer(x[name], flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                xp = {n: (None if t is None else t.copy()) for n, t in x.items()}
                xm = {n: (None if t is None else t.copy()) for n, t in x.items()}
                xp[name][idx] += eps
                xm[name][idx] -= eps
                gnum[idx] = (loss(xp) - loss(xm)) / (2 * eps)
            got = grads["d" + name]
            assert rel(got, gnum) < 1e-6, f"{kind} d{name}: rel err {rel(got, gnum):.2e}"


def pin_backward_retention_closed_form(bwd):
    """Scalar-decay linear attention with a constant per-head decay is
    o = (Q K^T .* D) V, D_nm = gamma^(n-m) for n >= m ("07 · linear 路线（二）",
    section 1): dv = (Q K^T .* D)^T do, dq = (do V^T .* D) K,
    dk = (do V^T .* D)^T Q."""
    r = np.random.default_rng(63)
    B, T, H, D = 1, 40, 2, 5
    q, k, v, do = (r.standard_normal((B, T, H, D)) for _ in range(4))
    gam = np.array([0.9, 0.97])
    g = np.broadcast_to(np.log(gam)[None, None, :], (B, T, H)).copy()
    res = bwd("decay_la", q, k, v, g, None, None, do, None)
    n = np.arange(T)
    for h in range(H):
        Dm = np.where(n[:, None] >= n[None, :], gam[h] ** np.maximum(n[:, None] - n[None, :], 0), 0.0)
        Q, K, V, dO = q[0, :, h], k[0, :, h], v[0, :, h], do[0, :, h]
        P = (Q @ K.T) * Dm
        G = (dO @ V.T) * Dm
        assert rel(res["o"][0, :, h], P @ V) < 1e-12
        assert rel(res["dv"][0, :, h], P.T @ dO) < 1e-12
        assert rel(res["dq"][0, :, h], G @ K) < 1e-12
        assert rel(res["dk"][0, :, h], G.T @ Q) < 1e-12


def pin_prologue_backward_fd(pro, rec, bwd):
    """The prologue's chain rule (pro.apply_backward on top of the core
    backward ``bwd``) against central finite differences of
    L = <do, o> + <dhT, hT> through the prologue followed by the recurrence,
    with respect to every raw input and parameter."""
    eps = 1e-6
    r = np.random.default_rng(65)
    B, T, H, Dk, Dv = 1, 5, 2, 3, 4
    for kind, opts in (("gdn", dict(qk_l2norm=True, scale=0.7, beta_sigmoid=True, beta_x2=True)),
                       ("kda", dict(qk_l2norm=True, scale=1.3, beta_sigmoid=True)),
                       ("decay_la", dict(qk_l2norm=True, scale=0.9))):
        x = dict(q=r.standard_normal((B, T, H, Dk)) * 2, k=r.standard_normal((B, T, H, Dk)) * 2,
                 v=r.standard_normal((B, T, H, Dv)),
                 g=(np.log(r.uniform(0.6, 0.99, (B, T, H, Dk))) if kind == "kda"
                    else r.standard_normal((B, T, H))),
                 beta=None if kind == "decay_la" else r.standard_normal((B, T, H)),
                 A_log=None if kind == "kda" else np.log(r.uniform(0.2, 2.0, H)),
                 dt_bias=None if kind == "kda" else r.standard_normal(H))
        h0 = r.standard_normal((B, H, Dv, Dk)) * 0.3
        do, dhT = r.standard_normal((B, T, H, Dv)), r.standard_normal((B, H, Dv, Dk))

        def prep(xx):
            return pro.apply(kind, xx["q"], xx["k"], xx["g"], xx["beta"], A_log=xx["A_log"], dt_bias=xx["dt_bias"],
                             **opts)

        def loss(xx):
            q2, k2, g2, b2 = prep(xx)
            o, hT = rec(kind, q2, k2, xx["v"], g2, b2, h0)
            return float(np.sum(o * do) + np.sum(hT * dhT))

        q2, k2, g2, b2 = prep(x)
        core = bwd(kind, q2, k2, x["v"], g2, b2, h0, do, dhT)
        got = pro.apply_backward(kind, x["q"], x["k"], x["g"], x["beta"], core["dq"], core["dk"], core["dg"],
                                 core["dbeta"], A_log=x["A_log"], dt_bias=x["dt_bias"], **opts)
        for name, key in (("q", "dq"), ("k", "dk"), ("g", "dg"), ("beta", "dbeta"), ("A_log", "dA_log"),
                          ("dt_bias", "ddt_bias")):
            if x[name] is None:
                continue
            gnum = np.zeros_like(x[name])
            it = np.nditer(x[name], flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                xp = {n: (None if t is None else t.copy()) for n, t in x.items()}
                xm = {n: (None if t is None else t.copy()) for n, t in x.items()}
                xp[name][idx] += eps
                xm[name][idx] -= eps
                gnum[idx] = (loss(xp) - loss(xm)) / (2 * eps)
            assert rel(got[key], gnum) < 1e-6, f"{kind} {key}: rel err {rel(got[key], gnum):.2e}"
