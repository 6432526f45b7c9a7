"""GPU: the differentiable entry point chunk_delta_rule, through
torch.autograd, for the dense and packed layouts, with and without the
prologue.

Every gradient the library returns is reproducible (its reductions add in
a fixed order), so each must equal, bit for bit, that of the library's
backward called directly with the same cotangents: a wrong tensor or
cotangent in the autograd plumbing fails that check.  dg and dbeta are also
compared with the fp64 oracle (the reverse sweep, and for the prologue its
chain rule) at the tolerances of the backward parity tests.  The per-head
sums dA_log and ddt_bias are checked against the fp64 sums of the
per-token terms the library itself returns, to fp32 summation error, and
against the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle.backward import recurrence_backward
from delta_rule_rnn_amd.inputs import Workload, generate, generate_raw

from .test_gpu_parity import assert_close_grad, to_dev

pytestmark = pytest.mark.gpu
EXACT = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


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
    leaf_of = {"dq": "q", "dk": "k", "dv": "v", "dg": "g", "dbeta": "beta", "dh0": "h0"}
    for n in EXACT:
        if grads[n] is None:
            assert leaves[leaf_of[n]] is None
            continue
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
    pairs = [("dq", "q"), ("dk", "k"), ("dv", "v"), ("dg", "g"), ("dbeta", "beta"), ("dh0", "h0")]
    if gate:
        pairs += [("dA_log", "A_log"), ("ddt_bias", "dt_bias")]
    for n, leaf in pairs:
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
        # the reduction itself: ddt_bias[h] adds the per-token raw-gate
        # gradients the library returns in dg (da_t), and dA_log[h] the terms
        # g^_t dg^_t = softplus(a_t + dt_h) / sigmoid(a_t + dt_h) * da_t.
        # Against their fp64 sums the only error is fp32 summation over T
        # terms: 64 eps_f32 sum_t |term_t| bounds it with room to spare.
        a = raw["g"][0].double().numpy() + raw["dt_bias"].double().numpy()[None, :]    # [T, H]
        da = dg_got[0].astype(np.float64)                                               # [T, H]
        sp = np.logaddexp(0.0, a)
        sig = 1.0 / (1.0 + np.exp(-a))
        eps = float(np.finfo(np.float32).eps)
        for name, leaf, terms in (("ddt_bias", "dt_bias", da), ("dA_log", "A_log", sp / sig * da)):
            val = leaves[leaf].grad.double().cpu().numpy()
            exact = terms.sum(axis=0)
            bound = 64 * eps * np.abs(terms).sum(axis=0)
            assert np.all(np.abs(val - exact) <= bound), f"{kind} {name}: {val} vs fp64 sum {exact}, bound {bound}"
        # and the whole chain against the oracle: the bf16 tolerance times
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


@pytest.mark.parametrize("kind,dt,pro", [("kda", "bf16", False), ("gdn", "f32", False), ("gdn", "bf16", True)])
def test_backward_is_reproducible(kind, dt, pro):
    """Two calls of the backward (dense; and packed through the prologue
    with gate generation) with the same arguments return bit-identical
    gradients, dbeta, dg, dA_log and ddt_bias included."""
    dra = _ops()
    w = Workload(f"{kind}_rep", kind, dt, B=2, H=3, T=300, Dk=64, Dv=64, h0_std=0.2, seed=98)
    if pro:
        x = generate_raw(w)
        d = to_dev(x)
        P = dra.Prologue(qk_l2norm=True, scale=0.5, beta_sigmoid=True, A_log=d["A_log"], dt_bias=d["dt_bias"])
    else:
        d = to_dev(generate(w))
        P = None
    gen = torch.Generator().manual_seed(99)
    do = torch.randn(d["v"].shape, generator=gen).to(d["v"].dtype).to("cuda:0")
    dhT = (torch.randn(d["h0"].shape, generator=gen) * 0.1).to("cuda:0")
    run = lambda: dra.backward(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], do, dhT, prologue=P)
    r1, r2 = run(), run()
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(r1, r2)):
        assert (a is None) == (b is None)
        if a is not None:
            assert torch.equal(a, b), f"result {i} differs between calls"
    if pro:
        cu = torch.tensor([0, 170, 170, 300], dtype=torch.int32, device="cuda:0")
        sq = lambda t: t[:1].reshape(t.shape[1:]).contiguous()
        h0p = torch.zeros(3, 3, 64, 64, device="cuda:0")
        runp = lambda: dra.backward_varlen(kind, sq(d["q"]), sq(d["k"]), sq(d["v"]), sq(d["g"]), sq(d["beta"]), cu,
                                           h0p, sq(do), None, prologue=P)
        p1, p2 = runp(), runp()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(p1, p2)):
            if a is not None:
                assert torch.equal(a, b), f"packed result {i} differs between calls"
