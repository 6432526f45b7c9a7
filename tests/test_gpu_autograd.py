"""GPU: the differentiable entry point chunk_delta_rule, through
torch.autograd, for the dense and packed layouts, with and without the
prologue.

dq, dk, dv and the state gradients are deterministic: they must equal, bit
for bit, those of the library's backward called directly with the same
cotangents.  dbeta, dg and the per-head parameter gradients add per-wave
partials with atomics in no fixed order, so two calls may differ by fp32
reassociation, which cancellation inside those sums can make large next to
the result.  They are compared with the fp64 oracle instead (the reverse
sweep, and for the prologue its chain rule), at the tolerances of the
backward parity tests: a wrong tensor or cotangent in the autograd plumbing
fails either check.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle.backward import recurrence_backward
from delta_rule_rnn_amd.inputs import Workload, generate, generate_raw

from .test_gpu_parity import assert_close_grad, to_dev

pytestmark = pytest.mark.gpu
EXACT = ("dq", "dk", "dv", "dh0")


def _ops():
    import delta_rule_rnn_amd as dra
    return dra


def _cpu(t):
    return None if t is None else t.detach().float().cpu()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("kind", ["kda", "gdn", "decay_la"])
def test_autograd_dense_matches_backward(kind, dt):
    dra = _ops()
    w = Workload(f"{kind}_ag", kind, dt, B=2, H=2, T=150, Dk=64, Dv=64, h0_std=0.2, seed=91)
    x = generate(w)
    d = to_dev(x)
    names = ["q", "k", "v", "g", "beta", "h0"]
    leaves = {n: (d[n].clone().requires_grad_(True) if d[n] is not None else None) for n in names}
    o, hT = dra.chunk_delta_rule(kind, leaves["q"], leaves["k"], leaves["v"], leaves["g"], leaves["beta"],
                                 initial_state=leaves["h0"], output_final_state=True)
    gen = torch.Generator().manual_seed(92)
    w1 = torch.randn(o.shape, generator=gen).to("cuda:0")
    w2 = (torch.randn(hT.shape, generator=gen) * 0.1).to("cuda:0")
    ((o.float() * w1).sum() + (hT * w2).sum()).backward()
    do = w1.to(o.dtype).contiguous()
    ref = dra.backward(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], do, w2)
    torch.cuda.synchronize()
    grads = dict(zip(["dq", "dk", "dv", "dg", "dbeta", "dh0"], ref))
    leaf_of = {"dq": "q", "dk": "k", "dv": "v", "dh0": "h0"}
    for n in EXACT:
        assert torch.equal(leaves[leaf_of[n]].grad, grads[n]), n
    orc = recurrence_backward(kind, x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"].transpose(-1, -2),
                              _cpu(do), _cpu(w2).transpose(-1, -2))
    assert_close_grad(leaves["g"].grad.float().cpu().numpy(), orc["dg"], dt, f"{kind} {dt} autograd dg")
    if kind == "decay_la":
        assert grads["dbeta"] is None and leaves["beta"] is None
    else:
        assert_close_grad(leaves["beta"].grad.float().cpu().numpy(), orc["dbeta"], dt, f"{kind} {dt} autograd dbeta")


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
    from oracle import prologue as opro
    dra = _ops()
    lengths = [90, 0, 64, 33]
    T, H, D, N = sum(lengths), 2, 64, len(lengths)
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    w = Workload(f"{kind}_ag_pk", kind, "bf16", B=1, H=H, T=T, Dk=D, Dv=D, seed=95)
    raw = generate_raw(w)
    x = to_dev(raw)
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda:0")
    h0 = (torch.randn(N, H, D, D, generator=torch.Generator().manual_seed(96)) * 0.2).to("cuda:0")
    gate = x["A_log"] is not None
    sq = lambda t: t[0].contiguous()
    leaves = {"q": sq(x["q"]), "k": sq(x["k"]), "v": sq(x["v"]), "g": sq(x["g"]), "beta": sq(x["beta"]), "h0": h0}
    if gate:
        leaves["A_log"], leaves["dt_bias"] = x["A_log"], x["dt_bias"]
    leaves = {n: t.clone().requires_grad_(True) for n, t in leaves.items()}
    mk = lambda src: dra.Prologue(qk_l2norm=True, scale=0.125, beta_sigmoid=True,
                                  A_log=src.get("A_log"), dt_bias=src.get("dt_bias"))
    o, hT = dra.chunk_delta_rule(kind, leaves["q"], leaves["k"], leaves["v"], leaves["g"], leaves["beta"],
                                 initial_state=leaves["h0"], output_final_state=True, cu_seqlens=cu_t,
                                 prologue=mk(leaves))
    gen = torch.Generator().manual_seed(97)
    w1 = torch.randn(o.shape, generator=gen).to("cuda:0")
    w2 = (torch.randn(hT.shape, generator=gen) * 0.1).to("cuda:0")
    ((o.float() * w1).sum() + (hT * w2).sum()).backward()
    plain = {n: t.detach() for n, t in leaves.items()}
    do = w1.to(o.dtype).contiguous()
    ref = dra.backward_varlen(kind, plain["q"], plain["k"], plain["v"], plain["g"], plain["beta"], cu_t, plain["h0"],
                              do, w2, prologue=mk(plain))
    torch.cuda.synchronize()
    grads = dict(zip(["dq", "dk", "dv", "dg", "dbeta", "dh0", "dA_log", "ddt_bias"], ref))
    for n, leaf in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dh0", "h0")):
        assert torch.equal(leaves[leaf].grad, grads[n]), n
    if not gate:
        assert grads["dA_log"] is None and grads["ddt_bias"] is None

    # the oracle: prologue, reverse sweep per sequence, chain rule back
    ok = dict(qk_l2norm=True, scale=0.125, beta_sigmoid=True,
              A_log=raw["A_log"] if gate else None, dt_bias=raw["dt_bias"] if gate else None)
    q2, k2, g2, b2 = opro.apply(kind, raw["q"], raw["k"], raw["g"], raw["beta"], **ok)
    do_c, w2_c, h0_c = _cpu(do)[None], _cpu(w2), _cpu(h0)
    core_dg = np.zeros_like(g2)
    dg_got = leaves["g"].grad.float().cpu().numpy()[None]
    db_got = leaves["beta"].grad.float().cpu().numpy()[None]
    for i in range(N):
        a, b = cu[i], cu[i + 1]
        if a == b:
            continue
        sl = lambda t: np.ascontiguousarray(t[:, a:b])
        core = recurrence_backward(kind, sl(q2), sl(k2), raw["v"][:, a:b], sl(g2), sl(b2),
                                   h0_c[i:i + 1].transpose(-1, -2), do_c[:, a:b], w2_c[i:i + 1].transpose(-1, -2))
        core_dg[:, a:b] = core["dg"]
        sr = lambda t: t[:, a:b]
        r = opro.apply_backward(kind, sr(raw["q"]), sr(raw["k"]), sr(raw["g"]), sr(raw["beta"]), core["dq"],
                                core["dk"], core["dg"], core["dbeta"], **ok)
        assert_close_grad(dg_got[:, a:b], r["dg"], "bf16", f"{kind} autograd seq {i} dg")
        assert_close_grad(db_got[:, a:b], r["dbeta"], "bf16", f"{kind} autograd seq {i} dbeta")
    if gate:
        # per-head sums over every token, held to the bf16 tolerance times
        # sum_t |coef_t| * max_t |dg^_t| (the size of the terms they add)
        full = opro.apply_backward(kind, raw["q"], raw["k"], raw["g"], raw["beta"], np.zeros_like(q2),
                                   np.zeros_like(k2), core_dg, None, **ok)
        gh = opro.scalar_gate(raw["g"], raw["A_log"], raw["dt_bias"])
        coef_dt = -np.exp(opro._f64(raw["A_log"])) * opro.sigmoid(opro._f64(raw["g"]) + opro._f64(raw["dt_bias"]))
        dgmax = np.max(np.abs(core_dg), axis=(0, 1))
        for name, leaf, coef in (("dA_log", "A_log", gh), ("ddt_bias", "dt_bias", coef_dt)):
            val = leaves[leaf].grad.float().cpu().numpy()
            scale = np.sum(np.abs(coef), axis=(0, 1)) * dgmax
            err = np.abs(val - full[name])
            assert np.all(err <= 2e-2 * scale), f"{kind} autograd {name}: |err| {err} > 2e-2 * {scale}"
