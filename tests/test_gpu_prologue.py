"""GPU parity of the fused input prologue (dr_forward / dr_forward_varlen /
dr_decode with a dr_prologue, through the C ABI): raw projections in, the
fp64 oracle's prologue (oracle/prologue.py) followed by its recurrence as the
reference.  Page: "Gated DeltaNet", sections "门控与 Head 映射" and "加载 Token
与写入系数".

Tolerances as for the plain forward: fp32 I/O max-rel 1e-4; bf16 I/O rel-L2
and max-rel 2e-2 (the kernels normalise the bf16 inputs in fp32 and round
the scaled operands once, where the plain path rounds them once too).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle import prologue as opro
from delta_rule_rnn_amd.inputs import Workload, generate, generate_raw

from .test_gpu_parity import assert_close, to_dev

pytestmark = pytest.mark.gpu


def _ops():
    import delta_rule_rnn_amd as dra
    return dra


def _pro(dra, x, d, qk=True, scale=1.0, sig=True, x2=False, gate=True, bias=True):
    """(GPU Prologue, oracle keyword arguments) for the same options."""
    gate = gate and x["A_log"] is not None
    gp = dra.Prologue(qk_l2norm=qk, scale=scale, beta_sigmoid=sig and x["beta"] is not None,
                      beta_x2=x2 and sig and x["beta"] is not None,
                      A_log=d["A_log"] if gate else None, dt_bias=d["dt_bias"] if gate and bias else None)
    ok = dict(qk_l2norm=qk, scale=scale, beta_sigmoid=gp.beta_sigmoid, beta_x2=gp.beta_x2,
              A_log=x["A_log"] if gate else None, dt_bias=x["dt_bias"] if gate and bias else None)
    return gp, ok


def _oracle(kind, x, ok, sl=lambda t: t, h0=None):
    q, k, g, b = opro.apply(kind, sl(x["q"]), sl(x["k"]), sl(x["g"]), None if x["beta"] is None else sl(x["beta"]),
                            **ok)
    return oracle.recurrence(kind, q, k, sl(x["v"]), g, b, h0)


FWD_CASES = [
    ("kda", "bf16", 128, dict(scale=0.5)),
    ("kda", "f32", 64, dict(x2=True, scale=1.7)),
    ("gdn", "bf16", 128, dict()),
    ("gdn", "f32", 64, dict(x2=True, bias=False)),
    ("gdn", "bf16", 64, dict(qk=False, sig=False, gate=False, scale=0.25)),   # scale alone (plain inputs)
    ("decay_la", "bf16", 128, dict(scale=0.125)),
    ("decay_la", "f32", 64, dict(qk=False)),
]


@pytest.mark.parametrize("kind,dt,D,opts", FWD_CASES, ids=lambda c: str(c))
def test_forward_prologue_matches_oracle(kind, dt, D, opts):
    dra = _ops()
    w = Workload(f"{kind}_raw", kind, dt, B=2, H=3, T=150, Dk=D, Dv=D, h0_std=0.1, seed=51)
    if opts.get("qk", True) or opts.get("sig", True) or opts.get("gate", True):
        x = generate_raw(w)
    else:
        # no normalisation, sigmoid or gate generation: the inputs must already
        # be the recurrence's (unit keys, beta in (0, 1), gates <= 0)
        x = dict(generate(w), A_log=None, dt_bias=None)
    d = to_dev(x)
    gp, ok = _pro(dra, x, d, **opts)
    o, hT = dra.forward(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], prologue=gp)
    torch.cuda.synchronize()
    ro, rs = _oracle(kind, x, ok, h0=x["h0"].transpose(-1, -2).contiguous())
    assert_close(o.float().cpu().numpy(), ro, dt, f"{kind} {dt} D{D} {opts} output")
    assert_close(hT.cpu().numpy(), np.swapaxes(rs, -1, -2), dt, f"{kind} {dt} D{D} {opts} state")


def test_forward_prologue_identity_is_plain_path():
    """A prologue that does nothing (no ops, scale 1) runs the plain kernels:
    bit-identical to the call without one."""
    dra = _ops()
    w = Workload("gdn_plain", "gdn", "bf16", B=1, H=2, T=200, Dk=128, Dv=128, seed=52)
    d = to_dev(generate(w))
    o1, h1 = dra.forward("gdn", d["q"], d["k"], d["v"], d["g"], d["beta"])
    o2, h2 = dra.forward("gdn", d["q"], d["k"], d["v"], d["g"], d["beta"], prologue=dra.Prologue())
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all() and torch.isfinite(h1).all()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


@pytest.mark.parametrize("kind", ["kda", "gdn", "decay_la"])
def test_varlen_prologue_matches_oracle(kind):
    dra = _ops()
    lengths = [100, 0, 64, 37, 129]
    T = sum(lengths)
    w = Workload(f"{kind}_raw_packed", kind, "bf16", B=1, H=2, T=T, Dk=128, Dv=128, seed=53)
    x = generate_raw(w)
    d = to_dev(x)
    gp, ok = _pro(dra, x, d, scale=0.75)
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda:0")
    sq = lambda t: None if t is None else t[0]
    o, hT = dra.forward_varlen(kind, sq(d["q"]), sq(d["k"]), sq(d["v"]), sq(d["g"]), sq(d["beta"]), cu_t,
                               prologue=gp)
    torch.cuda.synchronize()
    o, hT = o.float().cpu().numpy(), hT.cpu().numpy()
    for i, n in enumerate(lengths):
        a, b = cu[i], cu[i + 1]
        sl = lambda t: t[:, a:b].contiguous()
        ro, rs = _oracle(kind, x, ok, sl)
        if n > 0:
            assert_close(o[a:b][None], ro, "bf16", f"{kind} sequence {i} (length {n}) output")
        assert_close(hT[i:i + 1], np.swapaxes(rs, -1, -2), "bf16", f"{kind} sequence {i} state",
                     tol_max=2e-2 if n > 0 else 0.0)


DEC_CASES = [(kind, dt, D) for kind in ("kda", "gdn", "decay_la") for dt in ("f32", "bf16") for D in (64, 128)]


@pytest.mark.parametrize("kind,dt,D", DEC_CASES, ids=lambda c: str(c))
def test_decode_prologue_matches_oracle(kind, dt, D):
    dra = _ops()
    w = Workload(f"{kind}_raw_dec", kind, dt, B=2, H=3, T=4, Dk=D, Dv=D, h0_std=0.5, seed=54)
    x = generate_raw(w)
    d = to_dev(x)
    gp, ok = _pro(dra, x, d, x2=(kind == "gdn"), scale=0.9)
    state = d["h0"].clone()
    o = dra.decode(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], state, prologue=gp)
    torch.cuda.synchronize()
    ro, rs = _oracle(kind, x, ok, h0=x["h0"].transpose(-1, -2).contiguous())
    assert_close(o.float().cpu().numpy(), ro, dt, f"{kind} {dt} D{D} decode output")
    assert_close(state.cpu().numpy(), np.swapaxes(rs, -1, -2), "f32", f"{kind} {dt} D{D} decode state")


@pytest.mark.parametrize("kind", ["gdn", "decay_la"])
def test_prefill_then_decode_with_prologue(kind):
    """Prefill with the prologue, then decode with it: one oracle pass over
    all tokens."""
    dra = _ops()
    T1, T2 = 130, 5
    w = Workload(f"{kind}_raw_cont", kind, "bf16", B=1, H=4, T=T1 + T2, Dk=128, Dv=128, seed=55)
    x = generate_raw(w)
    d = to_dev(x)
    gp, ok = _pro(dra, x, d)
    cut = lambda t, a, b: None if t is None else t[:, a:b].contiguous()
    _, hT = dra.forward(kind, cut(d["q"], 0, T1), cut(d["k"], 0, T1), cut(d["v"], 0, T1), cut(d["g"], 0, T1),
                        cut(d["beta"], 0, T1), prologue=gp)
    o2 = dra.decode(kind, cut(d["q"], T1, T1 + T2), cut(d["k"], T1, T1 + T2), cut(d["v"], T1, T1 + T2),
                    cut(d["g"], T1, T1 + T2), cut(d["beta"], T1, T1 + T2), hT, prologue=gp)
    torch.cuda.synchronize()
    ro, rs = _oracle(kind, x, ok)
    assert_close(o2.float().cpu().numpy(), ro[:, T1:], "bf16", f"{kind} decode after prefill, output")
    assert_close(hT.cpu().numpy(), np.swapaxes(rs, -1, -2), "bf16", f"{kind} decode after prefill, state")


def test_prologue_full_size_sampled():
    """GDN at the long workload's sizes (B=1, H=32, T=32768, d=128, bf16)
    from raw projections with the full prologue (bench.py --mode prologue):
    two sampled heads against the oracle's prologue and recurrence."""
    dra = _ops()
    from delta_rule_rnn_amd.inputs import WORKLOADS
    w = WORKLOADS["gdn_bf16_long"]
    x = generate_raw(w)
    d = to_dev(x)
    gp, ok = _pro(dra, x, d, scale=w.Dk ** -0.5)
    o, hT = dra.forward("gdn", d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], prologue=gp)
    torch.cuda.synchronize()
    o, hT = o.float().cpu().numpy(), hT.cpu().numpy()
    for h in (0, 21):
        sl = lambda t: t[:, :, h:h + 1].contiguous()
        okh = dict(ok, A_log=ok["A_log"][h:h + 1], dt_bias=ok["dt_bias"][h:h + 1])
        q2, k2, g2, b2 = opro.apply("gdn", sl(x["q"]), sl(x["k"]), sl(x["g"]), sl(x["beta"]), **okh)
        ro, rs = oracle.recurrence("gdn", q2, k2, sl(x["v"]), g2, b2)
        assert_close(o[:, :, h:h + 1], ro, "bf16", f"head {h} output")
        assert_close(hT[:, h:h + 1], np.swapaxes(rs, -1, -2), "bf16", f"head {h} state")
