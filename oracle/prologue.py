"""Input prologue of the gated delta rule, fp64 numpy -- TEST INFRASTRUCTURE ONLY.

The elementwise pre-pass that turns a layer's raw projections into the
recurrence's inputs, as the page "Gated DeltaNet" gives it:
  - write strength and gate of the layer forward (section "门控与 Head 映射"):
        beta = sigmoid(b),   g = -exp(A_log) * softplus(a + dt_bias)
    with A_log and dt_bias one value per head;
  - token loads of the recurrent kernel (section "加载 Token 与写入系数"):
    q and k divided by sqrt(sum of squares + 1e-6) over the key channels,
    then q multiplied by the output scale; beta optionally doubled after the
    sigmoid (write strengths in (0, 2)).
Each function is the plain definition, in fp64; apply_backward() is the
chain rule through apply().  Pinned by tests/test_oracle_pins.py (closed
forms, invariants, a Householder special case through the recurrence, and
finite differences of the prologue followed by the recurrence).
"""
from __future__ import annotations

from typing import Optional

import numpy as np

NORM_EPS = 1e-6


def _f64(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def l2_normalize(x, eps: float = NORM_EPS) -> np.ndarray:
    """x / sqrt(sum_d x_d^2 + eps) over the last axis."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def sigmoid(x) -> np.ndarray:
    """1 / (1 + e^-x)."""
    x = _f64(x)
    return 1.0 / (1.0 + np.exp(-x))


def softplus(x) -> np.ndarray:
    """log(1 + e^x), evaluated as logaddexp(0, x) so that large x does not
    overflow."""
    return np.logaddexp(0.0, _f64(x))


def scalar_gate(a, A_log, dt_bias=None) -> np.ndarray:
    """g[b, t, h] = -exp(A_log[h]) * softplus(a[b, t, h] + dt_bias[h])."""
    a, A_log = _f64(a), _f64(A_log)
    bias = np.zeros_like(A_log) if dt_bias is None else _f64(dt_bias)
    return -np.exp(A_log) * softplus(a + bias)


def apply(kind: str, q, k, g, beta=None, *, qk_l2norm: bool = False, scale: float = 1.0,
          beta_sigmoid: bool = False, beta_x2: bool = False, A_log=None, dt_bias=None):
    """The recurrence's (q, k, g, beta) from raw inputs, in fp64.

    q, k: [B,T,H,Dk]; g: [B,T,H,Dk] (kda) or [B,T,H]; beta: [B,T,H] or None.
    A_log (and dt_bias) given => g is the raw projection `a` of a scalar gate.
    """
    q, k, g, beta = _f64(q), _f64(k), _f64(g), _f64(beta)
    if qk_l2norm:
        q, k = l2_normalize(q), l2_normalize(k)
    q = q * scale
    if beta is not None and beta_sigmoid:
        beta = sigmoid(beta) * (2.0 if beta_x2 else 1.0)
    if A_log is not None:
        if kind == "kda":
            raise ValueError("gate generation is defined for scalar gates only")
        g = scalar_gate(g, A_log, dt_bias)
    return q, k, g, beta


def apply_backward(kind: str, q, k, g, beta, dq, dk, dg, dbeta, *, qk_l2norm: bool = False, scale: float = 1.0,
                   beta_sigmoid: bool = False, beta_x2: bool = False, A_log=None, dt_bias=None):
    """Chain rule through apply(): given the raw inputs and the gradients with
    respect to the recurrence's inputs (dq, dk, dg, dbeta, shapes of apply's
    outputs), return the gradients with respect to the raw inputs as a dict
    {dq, dk, dg, dbeta, dA_log, ddt_bias} (the last two None without gate
    generation; dbeta None without beta).  fp64, each step the derivative of
    the matching step of apply():
      y = x / n, n = sqrt(|x|^2 + eps):   dx = (dy - y (y . dy)) / n
      q_out = scale * y_q:                dy_q = scale * dq_out
      b_out = s * sigmoid(b):             db = s * sigmoid(b) (1 - sigmoid(b)) * db_out
      g = -exp(A_log) softplus(a + dt):   da = -exp(A_log) sigmoid(a + dt) * dg,
                                          dA_log = sum over tokens of g * dg,
                                          ddt = sum over tokens of da
    """
    q, k, g, beta = _f64(q), _f64(k), _f64(g), _f64(beta)
    dq, dk, dg, dbeta = _f64(dq), _f64(dk), _f64(dg), _f64(dbeta)
    out = {}
    dyq = dq * scale
    if qk_l2norm:
        def back(x, dy):
            n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + NORM_EPS)
            y = x / n
            return (dy - y * np.sum(y * dy, axis=-1, keepdims=True)) / n
        out["dq"], out["dk"] = back(q, dyq), back(k, dk)
    else:
        out["dq"], out["dk"] = dyq, dk
    if beta is not None and dbeta is not None and beta_sigmoid:
        s = sigmoid(beta)
        out["dbeta"] = (2.0 if beta_x2 else 1.0) * s * (1.0 - s) * dbeta
    else:
        out["dbeta"] = dbeta
    if A_log is not None:
        if kind == "kda":
            raise ValueError("gate generation is defined for scalar gates only")
        A_log = _f64(A_log)
        bias = np.zeros_like(A_log) if dt_bias is None else _f64(dt_bias)
        gout = scalar_gate(g, A_log, bias)
        da = -np.exp(A_log) * sigmoid(g + bias) * dg
        out["dg"] = da
        red = tuple(range(da.ndim - 1))
        out["dA_log"] = np.sum(gout * dg, axis=red)
        out["ddt_bias"] = np.sum(da, axis=red) if dt_bias is not None else None
    else:
        out["dg"] = dg
        out["dA_log"] = out["ddt_bias"] = None
    return out
