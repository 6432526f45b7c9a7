"""GPU parity on the method's degenerate inputs, forward, backward and decode,
each against the fp64 oracle on the same inputs:

  beta = 0        no write: the state only decays (S_t = S_{t-1} Diag(a_t))
  g = 0 (a = 1)   no decay: the ungated delta rule, or plain linear attention
                  for decay_la (pages "Gated DeltaNet", section "DeltaNet 与
                  Gated Delta Rule"; "TileLang 实战：KDA 从零到一--标量衰减",
                  section 1.1)
  beta = 2        with unit keys, I - 2 k k^T is a reflection: the largest
                  write strength the doubled sigmoid of the prologue reaches
  q = 0           every output is exactly zero
  v = 0, h0 = 0   the state stays zero and so does every output
  strong decay    scalar gates of -20 per token (a ~ 2e-9): decays that
                  underflow across a chunk, handled by the ratio form; dg,
                  about 1e-9 there, is held to the tolerance times max|dk|
                  (the size of the terms that cancel to give it)

Tolerances as in test_gpu_parity: fp32 I/O max-rel 1e-4, bf16 I/O rel-L2 and
max-rel 2e-2; exact zeros where the mathematics gives exact zeros.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle.backward import recurrence_backward
from delta_rule_rnn_amd.inputs import Workload, generate

from .test_gpu_parity import assert_close, assert_close_grad, to_dev

pytestmark = pytest.mark.gpu

KINDS = ["kda", "gdn", "decay_la"]


def _ops():
    import delta_rule_rnn_amd as dra
    return dra


def _inputs(kind, dt, D=64, T=150, B=1, H=2, seed=81, h0_std=0.2):
    w = Workload(f"{kind}_degenerate", kind, dt, B=B, H=H, T=T, Dk=D, Dv=D, h0_std=h0_std, seed=seed)
    return w, generate(w)


def _forward_check(kind, dt, x, what):
    dra = _ops()
    d = to_dev(x)
    o, hT = dra.forward(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    torch.cuda.synchronize()
    h0 = None if x["h0"] is None else x["h0"].transpose(-1, -2)
    ro, rs = oracle.recurrence(kind, x["q"], x["k"], x["v"], x["g"], x["beta"], h0)
    assert_close(o.float().cpu().numpy(), ro, dt, f"{what} output")
    assert_close(hT.cpu().numpy(), np.swapaxes(rs, -1, -2), dt, f"{what} state")
    return o, hT


def _backward_check(kind, dt, x, what, seed=82, dg_abs=False):
    dra = _ops()
    gen = torch.Generator().manual_seed(seed)
    B, T, H, D = x["q"].shape
    do = torch.randn(B, T, H, D, generator=gen).to(x["q"].dtype)
    dhT = torch.randn(B, H, D, D, generator=gen) * 0.1
    d = to_dev(x)
    res = dra.backward(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], do.to("cuda:0"),
                       dhT.to("cuda:0"))
    torch.cuda.synchronize()
    h0 = None if x["h0"] is None else x["h0"].transpose(-1, -2)
    ref = recurrence_backward(kind, x["q"], x["k"], x["v"], x["g"], x["beta"], h0, do, dhT.transpose(-1, -2))
    got = [None if t is None else t.float().cpu().numpy() for t in res]
    for name, val in zip(["dq", "dk", "dv"], got[:3]):
        assert_close_grad(val, ref[name], dt, f"{what} {name}")
    if dg_abs:
        # the chunk form reaches dg as a sum of O(|dk|) terms that cancel
        # exactly in exact arithmetic: held to the dtype's tolerance times
        # that scale, not to the (vanishing) size of dg itself
        tol = 1e-4 if dt == "f32" else 2e-2
        err = np.max(np.abs(got[3] - ref["dg"]))
        scale = np.max(np.abs(ref["dk"]))
        assert err <= tol * scale, f"{what} dg: max abs err {err:.3e} > {tol} * {scale:.3e}"
    else:
        assert_close_grad(got[3], ref["dg"], dt, f"{what} dg")
    if kind != "decay_la":
        assert_close_grad(got[4], ref["dbeta"], dt, f"{what} dbeta")
    assert_close_grad(got[5], np.swapaxes(ref["dh0"], -1, -2), dt, f"{what} dh0")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["kda", "gdn"])
def test_beta_zero_only_decays(kind, dt):
    """beta = 0: the output is the decayed initial state read out, and the
    final state is h0 times the product of the gates."""
    _, x = _inputs(kind, dt)
    x = dict(x, beta=torch.zeros_like(x["beta"]))
    _forward_check(kind, dt, x, f"{kind} {dt} beta=0")
    _backward_check(kind, dt, x, f"{kind} {dt} beta=0")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("kind", KINDS)
def test_no_decay(kind, dt):
    """g = 0 everywhere (a = 1)."""
    _, x = _inputs(kind, dt)
    x = dict(x, g=torch.zeros_like(x["g"]))
    _forward_check(kind, dt, x, f"{kind} {dt} g=0")
    _backward_check(kind, dt, x, f"{kind} {dt} g=0")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["kda", "gdn"])
def test_beta_two_reflection(kind, dt):
    """beta = 2 with unit keys (the workloads' keys are L2-normalised)."""
    _, x = _inputs(kind, dt)
    x = dict(x, beta=torch.full_like(x["beta"], 2.0))
    _forward_check(kind, dt, x, f"{kind} {dt} beta=2")
    _backward_check(kind, dt, x, f"{kind} {dt} beta=2")


@pytest.mark.parametrize("kind", KINDS)
def test_zero_queries_give_zero_output(kind):
    """q = 0: every output element is exactly zero; the state still matches
    the oracle."""
    dra = _ops()
    _, x = _inputs(kind, "bf16")
    x = dict(x, q=torch.zeros_like(x["q"]))
    d = to_dev(x)
    o, hT = dra.forward(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0
    ro, rs = oracle.recurrence(kind, x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"].transpose(-1, -2))
    assert_close(hT.cpu().numpy(), np.swapaxes(rs, -1, -2), "bf16", f"{kind} q=0 state")


@pytest.mark.parametrize("kind", KINDS)
def test_zero_values_and_state_stay_zero(kind):
    """v = 0 and h0 = 0: the state never leaves zero, so o and hT are exactly
    zero (forward and decode)."""
    dra = _ops()
    _, x = _inputs(kind, "f32", h0_std=0.0)
    x = dict(x, v=torch.zeros_like(x["v"]))
    d = to_dev(x)
    o, hT = dra.forward(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], None)
    state = torch.zeros(1, 2, 64, 64, device="cuda:0")
    od = dra.decode(kind, d["q"][:, :3], d["k"][:, :3], d["v"][:, :3], d["g"][:, :3],
                    None if d["beta"] is None else d["beta"][:, :3], state)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0 and torch.count_nonzero(hT).item() == 0
    assert torch.count_nonzero(od).item() == 0 and torch.count_nonzero(state).item() == 0


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["gdn", "decay_la"])
def test_strong_scalar_decay(kind, dt):
    """Scalar gates of -20 per token: a chunk's cumulative decay underflows
    (2^-1800), which the ratio form 2^(gamma_i - gamma_j), j <= i, never
    evaluates; the output is then the current token's own write."""
    _, x = _inputs(kind, dt)
    x = dict(x, g=torch.full_like(x["g"], -20.0))
    _forward_check(kind, dt, x, f"{kind} {dt} g=-20")
    _backward_check(kind, dt, x, f"{kind} {dt} g=-20", dg_abs=True)


@pytest.mark.parametrize("kind", KINDS)
def test_decode_degenerate(kind):
    """The decode step on beta = 0 (delta kinds) and g = 0, fp32, from a
    nonzero state, against the token recurrence."""
    dra = _ops()
    _, x = _inputs(kind, "f32", T=4)
    cases = [dict(g=torch.zeros_like(x["g"]))]
    if kind != "decay_la":
        cases.append(dict(beta=torch.zeros_like(x["beta"])))
    for mod in cases:
        y = dict(x, **mod)
        d = to_dev(y)
        state = d["h0"].clone()
        o = dra.decode(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], state)
        torch.cuda.synchronize()
        ro, rs = oracle.recurrence(kind, y["q"], y["k"], y["v"], y["g"], y["beta"], y["h0"].transpose(-1, -2))
        what = f"{kind} decode {sorted(mod)}"
        assert_close(o.cpu().numpy(), ro, "f32", f"{what} output")
        assert_close(state.cpu().numpy(), np.swapaxes(rs, -1, -2), "f32", f"{what} state")
