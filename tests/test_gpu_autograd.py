"""GPU: the differentiable entry point chunk_delta_rule gives, through
torch.autograd, exactly the gradients of the library's backward called
directly with the same cotangents (which the backward parity tests compare
with the fp64 oracle), for the dense and packed layouts, with and without
the prologue.  dq, dk, dv and the state gradients are bit-identical; dbeta,
dg and the per-head parameter gradients add per-wave partials with atomics
in no fixed order, so they are compared to fp32 reassociation (1e-5 of
their largest magnitude).
"""
from __future__ import annotations

import pytest
import torch

from delta_rule_rnn_amd.inputs import Workload, generate, generate_raw

from .test_gpu_parity import to_dev

pytestmark = pytest.mark.gpu
EXACT = ("dq", "dk", "dv", "dh0")


def _ops():
    import delta_rule_rnn_amd as dra
    return dra


def _same(name, a, b):
    if name in EXACT:
        assert torch.equal(a, b), name
    else:
        err = (a.float() - b.float()).abs().max().item()
        assert err <= 1e-5 * max(b.float().abs().max().item(), 1e-30), (name, err)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("kind", ["kda", "gdn", "decay_la"])
def test_autograd_dense_matches_backward(kind, dt):
    dra = _ops()
    w = Workload(f"{kind}_ag", kind, dt, B=2, H=2, T=150, Dk=64, Dv=64, h0_std=0.2, seed=91)
    d = to_dev(generate(w))
    names = ["q", "k", "v", "g", "beta", "h0"]
    leaves = {n: (d[n].clone().requires_grad_(True) if d[n] is not None else None) for n in names}
    o, hT = dra.chunk_delta_rule(kind, leaves["q"], leaves["k"], leaves["v"], leaves["g"], leaves["beta"],
                                 initial_state=leaves["h0"], output_final_state=True)
    gen = torch.Generator().manual_seed(92)
    w1 = torch.randn(o.shape, generator=gen).to("cuda:0")
    w2 = (torch.randn(hT.shape, generator=gen) * 0.1).to("cuda:0")
    ((o.float() * w1).sum() + (hT * w2).sum()).backward()
    ref = dra.backward(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], w1.to(o.dtype).contiguous(), w2)
    torch.cuda.synchronize()
    for n, r in zip(["dq", "dk", "dv", "dg", "dbeta", "dh0"], ref):
        leaf = leaves[{"dq": "q", "dk": "k", "dv": "v", "dg": "g", "dbeta": "beta", "dh0": "h0"}[n]]
        if leaf is None:
            assert r is None
            continue
        _same(n, leaf.grad, r)


def test_autograd_output_only():
    """Without the final state requested, its cotangent is absent (the
    backward takes dhT as zero)."""
    dra = _ops()
    w = Workload("gdn_ag_o", "gdn", "bf16", B=1, H=2, T=100, Dk=64, Dv=64, h0_std=0.0, seed=93)
    d = to_dev(generate(w))
    q = d["q"].clone().requires_grad_(True)
    o, hT = dra.chunk_delta_rule("gdn", q, d["k"], d["v"], d["g"], d["beta"])
    assert hT is None
    w1 = torch.randn(o.shape, generator=torch.Generator().manual_seed(94)).to("cuda:0")
    (o.float() * w1).sum().backward()
    ref = dra.backward("gdn", d["q"], d["k"], d["v"], d["g"], d["beta"], None, w1.to(o.dtype).contiguous(), None)
    torch.cuda.synchronize()
    assert torch.equal(q.grad, ref[0])


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_autograd_packed_with_prologue(kind):
    """Packed sequences (one empty) on raw projections through the prologue:
    gradients of every raw input, the per-sequence initial states and, for
    the scalar gate, A_log and dt_bias."""
    dra = _ops()
    lengths = [90, 0, 64, 33]
    T = sum(lengths)
    w = Workload(f"{kind}_ag_pk", kind, "bf16", B=1, H=2, T=T, Dk=64, Dv=64, seed=95)
    x = to_dev(generate_raw(w))
    cu = torch.tensor([0, 90, 90, 154, 187], dtype=torch.int32, device="cuda:0")
    N = len(lengths)
    h0 = (torch.randn(N, 2, 64, 64, generator=torch.Generator().manual_seed(96)) * 0.2).to("cuda:0")
    gate = x["A_log"] is not None
    sq = lambda t: t[0].contiguous()
    leaves = {"q": sq(x["q"]), "k": sq(x["k"]), "v": sq(x["v"]), "g": sq(x["g"]), "beta": sq(x["beta"]), "h0": h0}
    if gate:
        leaves["A_log"], leaves["dt_bias"] = x["A_log"], x["dt_bias"]
    leaves = {n: t.clone().requires_grad_(True) for n, t in leaves.items()}
    mk = lambda src: dra.Prologue(qk_l2norm=True, scale=0.125, beta_sigmoid=True,
                                  A_log=src.get("A_log"), dt_bias=src.get("dt_bias"))
    o, hT = dra.chunk_delta_rule(kind, leaves["q"], leaves["k"], leaves["v"], leaves["g"], leaves["beta"],
                                 initial_state=leaves["h0"], output_final_state=True, cu_seqlens=cu,
                                 prologue=mk(leaves))
    gen = torch.Generator().manual_seed(97)
    w1 = torch.randn(o.shape, generator=gen).to("cuda:0")
    w2 = (torch.randn(hT.shape, generator=gen) * 0.1).to("cuda:0")
    ((o.float() * w1).sum() + (hT * w2).sum()).backward()
    plain = {n: t.detach() for n, t in leaves.items()}
    ref = dra.backward_varlen(kind, plain["q"], plain["k"], plain["v"], plain["g"], plain["beta"], cu, plain["h0"],
                              w1.to(o.dtype).contiguous(), w2, prologue=mk(plain))
    torch.cuda.synchronize()
    pairs = [("dq", "q"), ("dk", "k"), ("dv", "v"), ("dg", "g"), ("dbeta", "beta"), ("dh0", "h0"),
             ("dA_log", "A_log"), ("ddt_bias", "dt_bias")]
    for (n, leaf), r in zip(pairs, ref):
        if leaf not in leaves:
            assert r is None
            continue
        if n in ("dA_log", "ddt_bias"):
            _same_head_sum(n, leaves[leaf].grad, r, ref[3], plain)
        else:
            _same(n, leaves[leaf].grad, r)


def _same_head_sum(name, a, b, dg, x):
    """dA_log and ddt_bias are per-head sums over every token of fp32 terms
    whose order the atomics do not fix: with the gate g^ = -exp(A_log)
    softplus(a + dt_bias), the token terms are dg_t (ddt_bias) and
    dg_t softplus(a_t + dt_bias) / sigmoid(a_t + dt_bias) (dA_log), dg the
    gradient of the raw gate input.  Two summation orders of n fp32 terms
    differ by at most about n eps sum|term|; with n in the hundreds that is
    1e-5 of sum|term| per head."""
    z = (x["g"] + x["dt_bias"]).float()
    terms = dg.float().abs()
    if name == "dA_log":
        terms = terms * torch.nn.functional.softplus(z) / torch.sigmoid(z)
    bound = 1e-5 * terms.sum(0)
    err = (a.float() - b.float()).abs()
    assert torch.all(err <= bound), (name, err.tolist(), bound.tolist())
