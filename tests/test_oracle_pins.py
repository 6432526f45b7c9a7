"""CPU tests that pin the oracle (oracle/recurrence.c and oracle/chunked.py)
to what the pages and the mathematics fix.  No GPU involved."""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from oracle import chunked
from tests import pins
from tests.pins import rel, rand_case


@pytest.mark.parametrize("pin", pins.ALL_RECURRENCE_PINS, ids=lambda p: p.__name__)
def test_recurrence_pin(pin):
    pin(oracle.recurrence)


def test_chunk_form_equals_recurrence():
    pins.pin_chunk_form_equals_recurrence(oracle.recurrence, chunked)


def test_segment_form_equals_recurrence_and_token_maps():
    pins.pin_segment_form(oracle.recurrence, chunked)


def test_printed_decay_tables():
    """[SD] section 2.2: alpha=0.5, C=4 gives gamma = (0.5, 0.25, 0.125,
    0.0625) and Gamma(4,1) = 0.125; the alpha=0.9 D and Gamma matrices.
    Checked through the chunked oracle's step a1 (log2 cumsum) and step a2
    (with one key channel and k = 1, K+ K-^T is exactly the ratio matrix)."""
    gold = pins.read_golden("sd_decay_tables.txt")
    C = 4
    for alpha, key in ((0.5, None), (0.9, "Gamma_alpha0.9")):
        g = np.full((1, C, 1), np.log(alpha))
        gam = chunked.chunk_log2_cumsum(g, C)[0, :, 0]
        if alpha == 0.5:
            np.testing.assert_allclose(np.exp2(gam), gold["gamma_alpha0.5"][0], rtol=1e-14)
        one = np.ones((1, C, 1, 1))
        prep = chunked.separable_prep(one, one, gam[None, :, None], C)
        full = prep["Kp"][0, :, 0] @ prep["Km"][0, :, 0].T        # D_ij = gamma_i / gamma_j
        Gam = np.tril(full)
        if alpha == 0.5:
            assert abs(Gam[3, 0] - gold["gamma41_alpha0.5"][0, 0]) < 1e-14
        else:
            np.testing.assert_allclose(full, gold["D_alpha0.9"], atol=6e-4)
            np.testing.assert_allclose(Gam, gold[key], atol=6e-4)
            assert np.all(np.triu(Gam, 1) == 0)


def test_separable_identity():
    """[KDA] 1.2: StrictLower(K+ K-^T)_ci = sum_d k_c[d] e^(gamma_c[d]-gamma_i[d]) k_i[d]
    for i < c (the page reports 1.94e-16 between the two); also
    tril(Q~ K-^T) = the same weighted inner product with q on the left."""
    r = np.random.default_rng(5)
    C, Dk = 16, 8
    k = r.standard_normal((1, C, 1, Dk))
    q = r.standard_normal((1, C, 1, Dk))
    g = np.log(r.uniform(0.9, 0.999, (1, C, 1, Dk)))
    gam = chunked.chunk_log2_cumsum(g, C)
    prep = chunked.separable_prep(q, k, gam, C)
    M = np.tril(prep["Kp"][0, :, 0] @ prep["Km"][0, :, 0].T, -1)
    Aqk = np.tril(prep["Qp"][0, :, 0] @ prep["Km"][0, :, 0].T)
    G = np.cumsum(g[0, :, 0], axis=0)          # natural-log units
    naive = np.zeros((C, C))
    naive_qk = np.zeros((C, C))
    for c in range(C):
        for i in range(c + 1):
            w = np.exp(G[c] - G[i])
            naive_qk[c, i] = np.sum(q[0, c, 0] * w * k[0, i, 0])
            if i < c:
                naive[c, i] = np.sum(k[0, c, 0] * w * k[0, i, 0])
    assert rel(M, naive) < 1e-14
    assert rel(Aqk, naive_qk) < 1e-14
    # chunk-end quantities: phi = e^(gamma_C), Kbar = k e^(gamma_C - gamma)
    assert rel(prep["phi"][0, 0, 0], np.exp(G[-1])) < 1e-14
    assert rel(prep["Kbar"][0, :, 0], k[0, :, 0] * np.exp(G[-1] - G)) < 1e-14


def test_local_cumsum_resets_per_chunk():
    """[EVO] 3.5 / [SD] section 0: the cumulative sum restarts in every chunk
    (including a ragged last chunk)."""
    r = np.random.default_rng(6)
    g = -r.uniform(0, 1, (2, 37, 3))
    gam = chunked.chunk_log2_cumsum(g, 8)
    for s in range(0, 37, 8):
        e = min(s + 8, 37)
        np.testing.assert_allclose(gam[:, s:e], np.cumsum(g[:, s:e], 1) / np.log(2), rtol=1e-14)
        np.testing.assert_allclose(gam[:, s], g[:, s] / np.log(2), rtol=1e-14)


def test_triangular_inverse_pins():
    """T = (I + A)^-1 for strictly lower A: equals the finite Neumann series
    sum_{n<C} (-A)^n ([DPLR] 4.1, the path-sum view of the inverse) and a
    textbook forward substitution (scipy solve_triangular)."""
    from scipy.linalg import solve_triangular

    r = np.random.default_rng(7)
    C = 64
    A = np.tril(r.standard_normal((C, C)) * 0.05, -1)
    T = np.linalg.inv(np.eye(C) + A)
    neu = np.zeros((C, C))
    P = np.eye(C)
    for _ in range(C):
        neu += P
        P = P @ (-A)
    assert np.max(np.abs(P)) == 0.0 or np.max(np.abs(P)) < 1e-300  # nilpotent: (-A)^C = 0
    assert rel(T, neu) < 1e-13
    assert rel(T, solve_triangular(np.eye(C) + A, np.eye(C), lower=True, unit_diagonal=True)) < 1e-13
    # the inverse the chunked oracle produces for a real chunk, same checks
    q, k, v, g, bt, _ = rand_case("kda", B=1, T=C, H=1, Dk=16, Dv=8, seed=8)
    res = chunked.chunk_forward("kda", q, k, v, g, bt, None, C)
    A2, T2 = res.A[0, :, 0], res.Tinv[0, :, 0]
    assert np.all(np.triu(A2) == 0)
    assert rel(T2, solve_triangular(np.eye(C) + A2, np.eye(C), lower=True, unit_diagonal=True)) < 1e-12


def test_beta_pairings():
    """[KDA] 3.2-3.3: A = diag(beta) M with W = T diag(beta) K+ (row beta) and
    A = M diag(beta) with W = diag(beta) T K+ (column beta) are both right;
    mixing them is wrong and, with random beta, shows up at the 1e-1 level
    (the page measured rel-L2 1.3e-1).  The mixed pairing is planted in the
    oracle's step a3 and must be caught by the comparison with the
    recurrence."""
    def col_beta(Kp, Km, V, beta):
        n = Kp.shape[0]
        A = np.tril(Kp @ Km.T, -1) * beta[None, :]
        T = np.linalg.inv(np.eye(n) + A)
        return A, T, beta[:, None] * (T @ Kp), beta[:, None] * (T @ V)

    def mixed(Kp, Km, V, beta):   # column-beta A with the row-beta application
        n = Kp.shape[0]
        A = np.tril(Kp @ Km.T, -1) * beta[None, :]
        T = np.linalg.inv(np.eye(n) + A)
        return A, T, T @ (beta[:, None] * Kp), T @ (beta[:, None] * V)

    q, k, v, g, bt, _ = rand_case("kda", B=2, T=12, H=2, Dk=4, Dv=4, seed=9)
    o, _ = oracle.recurrence("kda", q, k, v, g, bt)
    good = chunked.chunk_forward("kda", q, k, v, g, bt, None, 4).o
    good2 = chunked.chunk_forward("kda", q, k, v, g, bt, None, 4, ut=col_beta).o
    bad = chunked.chunk_forward("kda", q, k, v, g, bt, None, 4, ut=mixed).o
    l2 = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    assert l2(good, o) < 1e-13 and l2(good2, o) < 1e-13
    assert l2(bad, o) > 1e-2
    # invisible when beta is constant (the page's warning)
    btc = np.full_like(bt, 0.5)
    o_c, _ = oracle.recurrence("kda", q, k, v, g, btc)
    bad_c = chunked.chunk_forward("kda", q, k, v, g, btc, None, 4, ut=mixed).o
    assert l2(bad_c, o_c) < 1e-13


def test_value_slices_independent():
    """[KDA] 3.4: splitting d_v into blocks changes nothing (each value column
    of the state evolves on its own) -- the GPU path relies on this."""
    q, k, v, g, bt, h0 = rand_case("kda", B=1, T=20, H=2, Dk=4, Dv=8, seed=12, h0_std=0.5)
    o, s = oracle.recurrence("kda", q, k, v, g, bt, h0)
    for blk in (1, 2, 4):
        for j in range(0, 8, blk):
            oj, sj = oracle.recurrence("kda", q, k, v[..., j:j + blk], g, bt, h0[:, :, j:j + blk])
            assert rel(oj, o[..., j:j + blk]) < 1e-13 and rel(sj, s[:, :, j:j + blk]) < 1e-13


def test_empty_and_threads():
    q, k, v, g, bt, h0 = rand_case("gdn", B=2, T=0, H=2, Dk=4, Dv=3, seed=13, h0_std=1.0)
    o, s = oracle.recurrence("gdn", q, k, v, g, bt, h0)
    assert o.shape == (2, 0, 2, 3) and rel(s, h0) == 0.0
    q, k, v, g, bt, h0 = rand_case("gdn", B=3, T=9, H=3, Dk=4, Dv=3, seed=14)
    o1, s1 = oracle.recurrence("gdn", q, k, v, g, bt, nthreads=1)
    o4, s4 = oracle.recurrence("gdn", q, k, v, g, bt, nthreads=4)
    assert np.array_equal(o1, o4) and np.array_equal(s1, s4)


# --------------------------------------------------------------------------
# Planted mistakes: each is a plausible slip in the C oracle (dropped term,
# wrong sign, wrong index, transposed operand, gate on the wrong side).  A
# mutated copy is compiled into a temporary directory and the pins above must
# reject every one of them.
# --------------------------------------------------------------------------
MUTATIONS = {
    "beta_dropped_in_erase": ("S[(size_t)i * Dk + j] -= bt * Sk[i] * kt[j];",
                              "S[(size_t)i * Dk + j] -= Sk[i] * kt[j];"),
    "beta_dropped_in_write": ("S[(size_t)i * Dk + j] += bt * vt[i] * kt[j];",
                              "S[(size_t)i * Dk + j] += vt[i] * kt[j];"),
    "erase_sign": ("S[(size_t)i * Dk + j] -= bt * Sk[i] * kt[j];",
                   "S[(size_t)i * Dk + j] += bt * Sk[i] * kt[j];"),
    "gate_channel_reversed": ("a[j] = exp(J->g[row * Dk + j]);",
                              "a[j] = exp(J->g[row * Dk + (Dk - 1 - j)]);"),
    "readout_with_k": ("for (int j = 0; j < Dk; ++j) acc += S[(size_t)i * Dk + j] * qt[j];",
                       "for (int j = 0; j < Dk; ++j) acc += S[(size_t)i * Dk + j] * kt[j];"),
    "la_decay_after_write": ("S[(size_t)i * Dk + j] = a[j] * S[(size_t)i * Dk + j] + vt[i] * kt[j];",
                             "S[(size_t)i * Dk + j] = a[j] * (S[(size_t)i * Dk + j] + vt[i] * kt[j]);"),
    "gate_not_exponentiated": ("const double s = exp(J->g[row]);", "const double s = 1.0 + J->g[row];"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(os.path.join(os.path.dirname(oracle.__file__), "recurrence.c")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor not found: {name}"
    mut = src.replace(old, new)
    cpath = tmp_path / "mut.c"
    cpath.write_text(mut)
    so = str(tmp_path / "libmut.so")
    oracle.build(str(cpath), so)

    def rec(*a, **kw):
        return oracle.recurrence(*a, lib_path=so, **kw)

    caught = []
    for pin in pins.ALL_RECURRENCE_PINS:
        try:
            pin(rec)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"


# --------------------------------------------------------------------------
# Input prologue (oracle/prologue.py)
# --------------------------------------------------------------------------
from oracle import prologue as _prologue  # noqa: E402


@pytest.mark.parametrize("pin", pins.ALL_PROLOGUE_PINS, ids=lambda p: p.__name__)
def test_prologue_pin(pin):
    pin(_prologue)


def test_prologue_householder_through_recurrence():
    pins.pin_prologue_householder(_prologue, oracle.recurrence)


def test_prologue_gate_rejected_for_per_channel():
    with pytest.raises(ValueError):
        _prologue.apply("kda", np.ones((1, 1, 1, 4)), np.ones((1, 1, 1, 4)), np.zeros((1, 1, 1, 4)),
                        np.zeros((1, 1, 1)), A_log=np.zeros(1))


# Planted mistakes in the prologue: each must be caught by some prologue pin.
PROLOGUE_MUTATIONS = {
    "eps_outside_sqrt": ("x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)",
                         "x / (np.sqrt(np.sum(x * x, axis=-1, keepdims=True)) + eps)"),
    "norm_over_heads": ("return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)",
                        "return x / np.sqrt(np.sum(x * x, axis=-2, keepdims=True) + eps)"),
    "sigmoid_sign": ("1.0 / (1.0 + np.exp(-x))", "1.0 / (1.0 + np.exp(x))"),
    "softplus_as_log1p_of_x": ("np.logaddexp(0.0, _f64(x))", "np.log1p(np.abs(_f64(x)))"),
    "gate_without_exp": ("-np.exp(A_log) * softplus(a + bias)", "-A_log * softplus(a + bias)"),
    "gate_bias_dropped": ("softplus(a + bias)", "softplus(a)"),
    "scale_before_norm": ("    if qk_l2norm:\n        q, k = l2_normalize(q), l2_normalize(k)\n    q = q * scale\n",
                          "    q = q * scale\n    if qk_l2norm:\n        q, k = l2_normalize(q), l2_normalize(k)\n"),
    "beta_x2_ignored": ("sigmoid(beta) * (2.0 if beta_x2 else 1.0)", "sigmoid(beta)"),
}


@pytest.mark.parametrize("name", sorted(PROLOGUE_MUTATIONS))
def test_prologue_pins_catch_planted_mistake(name, tmp_path):
    import importlib.util
    src = open(_prologue.__file__).read()
    old, new = PROLOGUE_MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor not found: {name}"
    path = tmp_path / "prologue_mut.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("prologue_mut", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    caught = []
    for pin in pins.ALL_PROLOGUE_PINS:
        try:
            pin(mod)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no prologue pin caught the planted mistake {name}"


# --------------------------------------------------------------------------
# Backward pass (oracle/backward.py)
# --------------------------------------------------------------------------
from oracle import backward as _backward  # noqa: E402


def test_backward_finite_differences():
    pins.pin_backward_finite_differences(_backward.recurrence_backward, oracle.recurrence)


def test_backward_retention_closed_form():
    pins.pin_backward_retention_closed_form(_backward.recurrence_backward)


def test_backward_forward_matches_recurrence():
    """The forward the backward recomputes is the C oracle's."""
    for kind in ("kda", "gdn", "decay_la"):
        x, do, dhT = pins._fd_case(kind, 64)
        res = _backward.recurrence_backward(kind, x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], do, dhT)
        o, hT = oracle.recurrence(kind, x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
        assert rel(res["o"], o) < 1e-13 and rel(res["hT"], hT) < 1e-13


BACKWARD_MUTATIONS = {
    "dq_from_entry_state": ('out["dq"][b, t, h] = S[t + 1].T @ dot', 'out["dq"][b, t, h] = S[t].T @ dot'),
    "readout_adjoint_after_use": ("                dS += np.outer(dot, qt)\n", ""),
    "dv_without_beta": ('out["dv"][b, t, h] = beta[b, t, h] * dr', 'out["dv"][b, t, h] = dr'),
    "du_sign": ("du = -beta[b, t, h] * dr", "du = beta[b, t, h] * dr"),
    "dbeta_uses_v_only": ('out["dbeta"][b, t, h] = dr @ (v[b, t, h] - u)', 'out["dbeta"][b, t, h] = dr @ v[b, t, h]'),
    "dk_misses_read_term": ("dkt = dkt + Sbar.T @ du", "dkt = dkt"),
    "dg_without_a": ('out["dg"][b, t, h] = a * da if perch else a * np.sum(da)',
                     'out["dg"][b, t, h] = da if perch else np.sum(da)'),
    "gate_adjoint_not_decayed": ("                dS = dS * a\n", ""),
    "dg_from_exit_state": ("da = np.sum(dS * S[t], axis=0)", "da = np.sum(dS * S[t + 1], axis=0)"),
}


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTATIONS))
def test_backward_pins_catch_planted_mistake(name, tmp_path):
    import importlib.util
    src = open(_backward.__file__).read()
    old, new = BACKWARD_MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor not found: {name}"
    path = tmp_path / "backward_mut.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("backward_mut", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    caught = []
    for pin in (lambda f: pins.pin_backward_finite_differences(f, oracle.recurrence),
                pins.pin_backward_retention_closed_form):
        try:
            pin(mod.recurrence_backward)
        except AssertionError:
            caught.append(pin)
    assert caught, f"no backward pin caught the planted mistake {name}"


def test_prologue_backward_finite_differences():
    pins.pin_prologue_backward_fd(_prologue, oracle.recurrence, _backward.recurrence_backward)


PROLOGUE_BACKWARD_MUTATIONS = {
    "scale_dropped": ("    dyq = dq * scale\n", "    dyq = dq\n"),
    "projection_sign": ("return (dy - y * np.sum(y * dy, axis=-1, keepdims=True)) / n",
                        "return (dy + y * np.sum(y * dy, axis=-1, keepdims=True)) / n"),
    "sigmoid_derivative": ("(2.0 if beta_x2 else 1.0) * s * (1.0 - s) * dbeta", "(2.0 if beta_x2 else 1.0) * s * dbeta"),
    "gate_exp_dropped": ("da = -np.exp(A_log) * sigmoid(g + bias) * dg", "da = -sigmoid(g + bias) * dg"),
    "dA_log_without_g": ('out["dA_log"] = np.sum(gout * dg, axis=red)', 'out["dA_log"] = np.sum(dg, axis=red)'),
}


@pytest.mark.parametrize("name", sorted(PROLOGUE_BACKWARD_MUTATIONS))
def test_prologue_backward_pins_catch_planted_mistake(name, tmp_path):
    import importlib.util
    src = open(_prologue.__file__).read()
    old, new = PROLOGUE_BACKWARD_MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor not found: {name}"
    path = tmp_path / "prologue_bmut.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("prologue_bmut", str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with pytest.raises(AssertionError):
        pins.pin_prologue_backward_fd(mod, oracle.recurrence, _backward.recurrence_backward)
