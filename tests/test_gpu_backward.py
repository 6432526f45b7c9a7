"""GPU parity of the backward (dr_backward through the C ABI) against the
fp64 oracle's reverse sweep of the token recurrence (oracle/backward.py).
Page: "Gated DeltaNet", section "反向传播：状态伴随与三角变换梯度".

Tolerances: fp32 I/O max-rel 1e-4 for every gradient; bf16 I/O rel-L2 and
max-rel 2e-2 (the inputs are the same bf16 values on both sides; the kernels
compute in fp32 and round dq, dk, dv once to bf16 on the store; dg, dbeta
and dh0 are fp32 outputs).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle.backward import recurrence_backward
from delta_rule_rnn_amd.inputs import Workload, generate

from .test_gpu_parity import assert_close_grad, to_dev

pytestmark = pytest.mark.gpu


def _ops():
    import delta_rule_rnn_amd as dra
    return dra


def _cotangents(w, seed):
    gen = torch.Generator().manual_seed(seed)
    do = torch.randn(w.B, w.T, w.H, w.Dv, generator=gen)
    dhT = torch.randn(w.B, w.H, w.Dk, w.Dv, generator=gen) * 0.1
    return do, dhT


def _run(kind, dt, D, B, H, T, seed, with_h0=True, with_dhT=True):
    dra = _ops()
    w = Workload(f"{kind}_bwd", kind, dt, B=B, H=H, T=T, Dk=D, Dv=D, h0_std=0.2 if with_h0 else 0.0, seed=seed)
    x = generate(w)
    do, dhT = _cotangents(w, seed + 100)
    do = do.to(x["q"].dtype)
    dhT = dhT if with_dhT else None
    d = to_dev(x)
    res = dra.backward(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], do.to("cuda:0"),
                       None if dhT is None else dhT.to("cuda:0"))
    torch.cuda.synchronize()
    ref = recurrence_backward(kind, x["q"], x["k"], x["v"], x["g"], x["beta"],
                              None if x["h0"] is None else x["h0"].transpose(-1, -2), do,
                              None if dhT is None else dhT.transpose(-1, -2))
    return res, ref


def _check(res, ref, kind, dt, what):
    dq, dk, dv, dg, dbeta, dh0 = (None if t is None else t.float().cpu().numpy() for t in res)
    assert_close_grad(dq, ref["dq"], dt, f"{what} dq")
    assert_close_grad(dk, ref["dk"], dt, f"{what} dk")
    assert_close_grad(dv, ref["dv"], dt, f"{what} dv")
    assert_close_grad(dg, ref["dg"], "f32" if dt == "f32" else dt, f"{what} dg")
    if kind != "decay_la":
        assert_close_grad(dbeta, ref["dbeta"], dt, f"{what} dbeta")
    assert_close_grad(dh0, np.swapaxes(ref["dh0"], -1, -2), dt, f"{what} dh0")


CASES = [(kind, dt, D) for kind in ("kda", "gdn", "decay_la") for dt in ("f32", "bf16") for D in (64, 128)]


@pytest.mark.parametrize("kind,dt,D", CASES, ids=lambda c: str(c))
def test_backward_matches_oracle(kind, dt, D):
    """Three chunks, the last ragged (150 = 64 + 64 + 22), two batches and
    heads, an initial state and a final-state cotangent."""
    res, ref = _run(kind, dt, D, B=2, H=2, T=150, seed=71)
    _check(res, ref, kind, dt, f"{kind} {dt} D{D}")


@pytest.mark.parametrize("kind", ["kda", "gdn", "decay_la"])
@pytest.mark.parametrize("T", [1, 64, 65])
def test_backward_lengths(kind, T):
    """One token, exactly one chunk, one chunk plus one token (with an
    initial state, so that every gradient is nonzero)."""
    res, ref = _run(kind, "f32", 64, B=1, H=3, T=T, seed=72, with_h0=True, with_dhT=False)
    _check(res, ref, kind, "f32", f"{kind} T={T}")


@pytest.mark.parametrize("kind", ["kda", "gdn", "decay_la"])
def test_backward_zero_initial_state(kind):
    """No initial state and no final-state cotangent (h0 = dhT = NULL)."""
    res, ref = _run(kind, "bf16", 128, B=1, H=2, T=200, seed=75, with_h0=False, with_dhT=False)
    _check(res, ref, kind, "bf16", f"{kind} zero h0")


@pytest.mark.parametrize("path", ["segment", "slices"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["kda", "gdn", "decay_la"])
@pytest.mark.parametrize("B,H,T", [(1, 2, 2600), (2, 2, 8300)])
def test_backward_reverse_pass_paths(kind, D, path, B, H, T, monkeypatch):
    """bf16 I/O: the segment-parallel reverse pass (the default) and the
    value-slice kernel (DR_BWD_REV=slices), each against the oracle.  2 chains
    of 41 chunks give 41 one-chunk segments; 4 chains of 130 chunks (the last
    ragged) give 44 segments of 3 chunks, the last with one."""
    monkeypatch.setenv("DR_BWD_REV", path)
    res, ref = _run(kind, "bf16", D, B=B, H=H, T=T, seed=76)
    _check(res, ref, kind, "bf16", f"{kind} D{D} {path} T={T}")


@pytest.mark.parametrize("grad", ["bf16lds", "f32lds"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["kda", "gdn", "decay_la"])
def test_backward_gradient_kernel_paths(kind, D, grad, monkeypatch):
    """bf16 I/O: the gradient kernel with bf16 LDS operands (the default,
    with the bf16 prep that also writes the state pass's records) and the one
    with fp32 LDS operands (DR_BWD_GRAD=f32lds, with the forward's chunk
    kernel and the fp32-operand prep), each against the oracle: 2 batches
    of 3 chunks (the last ragged) and a 260-token chain of 5 chunks."""
    monkeypatch.setenv("DR_BWD_GRAD", grad)
    monkeypatch.delenv("DR_BWD_REV", raising=False)
    for (B, H, T, seed) in ((2, 2, 150, 81), (1, 3, 260, 82)):
        res, ref = _run(kind, "bf16", D, B=B, H=H, T=T, seed=seed)
        _check(res, ref, kind, "bf16", f"{kind} D{D} {grad} T={T}")


def test_backward_many_chains_one_segment(monkeypatch):
    """256 chains fill the GPU by themselves: the segment-parallel pass runs
    each chain as one segment (no maps, no composition)."""
    monkeypatch.delenv("DR_BWD_REV", raising=False)
    res, ref = _run("gdn", "bf16", 64, B=2, H=128, T=150, seed=77)
    _check(res, ref, "gdn", "bf16", "gdn 256 chains")


def test_backward_no_tokens():
    dra = _ops()
    w = Workload("gdn_bwd0", "gdn", "f32", B=2, H=2, T=0, Dk=64, Dv=64, h0_std=1.0, seed=73)
    d = to_dev(generate(w))
    dhT = torch.randn(2, 2, 64, 64, device="cuda:0")
    do = torch.empty(2, 0, 2, 64, device="cuda:0")
    _, _, _, _, _, dh0 = dra.backward("gdn", d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], do, dhT)
    _, _, _, _, _, dz = dra.backward("gdn", d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], do, None)
    torch.cuda.synchronize()
    assert torch.equal(dh0, dhT) and torch.count_nonzero(dz).item() == 0


def test_backward_long_sampled():
    """KDA bf16 d=128 over 1000 tokens (16 chunks): every gradient of two
    sampled (b, h) chains against the oracle run on those chains."""
    dra = _ops()
    w = Workload("kda_bwd_long", "kda", "bf16", B=1, H=6, T=1000, Dk=128, Dv=128, h0_std=0.1, seed=74)
    x = generate(w)
    do, dhT = _cotangents(w, 174)
    do = do.to(torch.bfloat16)
    d = to_dev(x)
    res = dra.backward("kda", d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], do.to("cuda:0"), dhT.to("cuda:0"))
    torch.cuda.synchronize()
    res = [t.float().cpu().numpy() for t in res]
    for h in (1, 4):
        sl = lambda t: t[:, :, h:h + 1].contiguous()
        ref = recurrence_backward("kda", sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]),
                                  x["h0"][:, h:h + 1].transpose(-1, -2), sl(do), dhT[:, h:h + 1].transpose(-1, -2))
        names = ["dq", "dk", "dv", "dg", "dbeta"]
        for n, r in zip(names, res[:5]):
            assert_close_grad(r[:, :, h:h + 1], ref[n], "bf16", f"head {h} {n}")
        assert_close_grad(res[5][:, h:h + 1], np.swapaxes(ref["dh0"], -1, -2), "bf16", f"head {h} dh0")


def test_backward_full_size_sampled():
    """The benchmark workload (KDA bf16, B=1, H=32, T=32768, d=128) through
    the same call bench.py --mode backward times; every gradient of three
    sampled heads (the first, one inside, the last: different workgroups of
    every launch) against the oracle run on each head alone."""
    dra = _ops()
    from delta_rule_rnn_amd.inputs import WORKLOADS
    w = WORKLOADS["kda_bf16_long"]
    x = generate(w)
    gen = torch.Generator().manual_seed(99)
    do = torch.randn(w.B, w.T, w.H, w.Dv, generator=gen).to(torch.bfloat16)
    dhT = torch.randn(w.B, w.H, w.Dk, w.Dv, generator=gen) * 0.1
    d = to_dev(x)
    res = dra.backward("kda", d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], do.to("cuda:0"), dhT.to("cuda:0"))
    torch.cuda.synchronize()
    res = [t.float().cpu().numpy() for t in res]
    for h in (0, 13, w.H - 1):
        sl = lambda t: t[:, :, h:h + 1].contiguous()
        ref = recurrence_backward("kda", sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]), None,
                                  sl(do), dhT[:, h:h + 1].transpose(-1, -2))
        for n, r in zip(["dq", "dk", "dv", "dg", "dbeta"], res[:5]):
            assert_close_grad(r[:, :, h:h + 1], ref[n], "bf16", f"full size head {h} {n}")
        assert_close_grad(res[5][:, h:h + 1], np.swapaxes(ref["dh0"], -1, -2), "bf16", f"full size head {h} dh0")


PRO_CASES = [("kda", "bf16", 128, dict(qk=True, sig=True, x2=False, scale=0.5)),
             ("kda", "f32", 64, dict(qk=True, sig=True, x2=True, scale=1.2)),
             ("gdn", "bf16", 128, dict(qk=True, sig=True, x2=False, scale=0.09)),
             ("gdn", "f32", 64, dict(qk=True, sig=True, x2=True, scale=1.0)),
             ("decay_la", "bf16", 64, dict(qk=True, sig=False, x2=False, scale=0.125)),
             ("decay_la", "f32", 128, dict(qk=False, sig=False, x2=False, scale=0.7))]


@pytest.mark.parametrize("kind,dt,D,opts", PRO_CASES, ids=lambda c: str(c))
def test_backward_through_prologue(kind, dt, D, opts):
    """Raw projections in (generate_raw): the backward through the prologue
    against the oracle's prologue chain rule on top of its reverse sweep of
    the prologue's outputs; dA_log and ddt_bias included for scalar gates."""
    from oracle import prologue as opro
    from delta_rule_rnn_amd.inputs import generate_raw
    dra = _ops()
    w = Workload(f"{kind}_bwd_pro", kind, dt, B=2, H=3, T=150, Dk=D, Dv=D, h0_std=0.2, seed=76)
    x = generate_raw(w)
    do, dhT = _cotangents(w, 176)
    do = do.to(x["q"].dtype)
    gate = x["A_log"] is not None
    if not opts["qk"]:
        # without the normalisation the raw keys must already be short enough
        # for a stable recurrence
        x = dict(x, k=(x["k"].float() * 0.02).to(x["k"].dtype))
    d = to_dev(x)
    pro = dra.Prologue(qk_l2norm=opts["qk"], scale=opts["scale"], beta_sigmoid=opts["sig"] and kind != "decay_la",
                       beta_x2=opts["x2"] and kind != "decay_la",
                       A_log=d["A_log"] if gate else None, dt_bias=d["dt_bias"] if gate else None)
    ok = dict(qk_l2norm=pro.qk_l2norm, scale=pro.scale, beta_sigmoid=pro.beta_sigmoid, beta_x2=pro.beta_x2,
              A_log=x["A_log"] if gate else None, dt_bias=x["dt_bias"] if gate else None)
    res = dra.backward(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], do.to("cuda:0"), dhT.to("cuda:0"),
                       prologue=pro)
    torch.cuda.synchronize()
    q2, k2, g2, b2 = opro.apply(kind, x["q"], x["k"], x["g"], x["beta"], **ok)
    core = recurrence_backward(kind, q2, k2, x["v"], g2, b2, x["h0"].transpose(-1, -2), do, dhT.transpose(-1, -2))
    ref = opro.apply_backward(kind, x["q"], x["k"], x["g"], x["beta"], core["dq"], core["dk"], core["dg"],
                              core["dbeta"], **ok)
    got = [None if t is None else t.float().cpu().numpy() for t in res]
    what = f"{kind} {dt} D{D} {opts}"
    assert_close_grad(got[0], ref["dq"], dt, f"{what} dq")
    assert_close_grad(got[1], ref["dk"], dt, f"{what} dk")
    assert_close_grad(got[2], core["dv"], dt, f"{what} dv")
    assert_close_grad(got[3], ref["dg"], dt, f"{what} dg")
    if kind != "decay_la":
        assert_close_grad(got[4], ref["dbeta"], dt, f"{what} dbeta")
    assert_close_grad(got[5], np.swapaxes(core["dh0"], -1, -2), dt, f"{what} dh0")
    if gate:
        # sums over all tokens of coef_t * dg^_t, with cancellation.  The
        # per-token dg^ is held to the dtype's tolerance relative to its
        # largest element, so the sum is held to that tolerance times
        # sum_t |coef_t| * max_t |dg^_t| (the same bound carried through the
        # sum)
        tol = 1e-4 if dt == "f32" else 2e-2
        gh = opro.scalar_gate(x["g"], x["A_log"], x["dt_bias"])
        coef_dt = -np.exp(opro._f64(x["A_log"])) * opro.sigmoid(opro._f64(x["g"]) + opro._f64(x["dt_bias"]))
        dgmax = np.max(np.abs(core["dg"]), axis=(0, 1))
        for name, val, coef in (("dA_log", got[6], gh), ("ddt_bias", got[7], coef_dt)):
            scale = np.sum(np.abs(coef), axis=(0, 1)) * dgmax
            err = np.abs(val - ref[name])
            assert np.all(err <= tol * scale), f"{what} {name}: |err| {err} > {tol} * {scale}"
    else:
        assert got[6] is None and got[7] is None
