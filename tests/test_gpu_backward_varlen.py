"""GPU parity of the packed-sequence backward (dr_backward_varlen through the
C ABI): each sequence's gradients against the fp64 oracle's reverse sweep
run on that sequence alone, equal lengths against the dense batched
backward (bit-identical: same chunks, same arithmetic), the backward through
the prologue, no tokens at all, and malformed offsets (flagged and clamped).
Page: "Gated DeltaNet", section "反向传播：状态伴随与三角变换梯度".

Tolerances as for the dense backward: fp32 I/O max-rel 1e-4, bf16 I/O
rel-L2 and max-rel 2e-2.
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


def _packed(kind, dt, D, lengths, seed, H=3):
    """Inputs of len(lengths) sequences drawn as one batch of T = sum tokens,
    per-sequence initial states and final-state cotangents, the output
    cotangent, and cu_seqlens as a list."""
    T = int(sum(lengths))
    w = Workload(f"{kind}_packed_bwd", kind, dt, B=1, H=H, T=T, Dk=D, Dv=D, seed=seed)
    x = generate(w)
    N = len(lengths)
    gen = torch.Generator().manual_seed(seed + 1)
    h0 = torch.randn(N, H, D, D, generator=gen) * 0.2
    dhT = torch.randn(N, H, D, D, generator=gen) * 0.1
    do = torch.randn(1, T, H, D, generator=gen).to(x["q"].dtype)
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return x, h0, dhT, do, cu


def _seq_ref(kind, x, h0, dhT, do, a, b, i):
    sl = lambda t: None if t is None else t[:, a:b].contiguous()
    return recurrence_backward(kind, sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]),
                               h0[i:i + 1].transpose(-1, -2), sl(do), dhT[i:i + 1].transpose(-1, -2))


def _check_seq(got, ref, kind, dt, a, b, i, what):
    dq, dk, dv, dg, dbeta, dh0 = got
    if b > a:
        for name, val in (("dq", dq), ("dk", dk), ("dv", dv), ("dg", dg)):
            assert_close_grad(val[:, a:b], ref[name], dt, f"{what} seq {i} {name}")
        if kind != "decay_la":
            assert_close_grad(dbeta[:, a:b], ref["dbeta"], dt, f"{what} seq {i} dbeta")
    assert_close_grad(dh0[i:i + 1], np.swapaxes(ref["dh0"], -1, -2), dt, f"{what} seq {i} dh0")


# bf16 I/O runs both reverse passes: the segment-parallel one (the default,
# one segment per sequence and head) and the value-slice one
CASES = [(kind, "bf16", 128, path) for kind in ("kda", "gdn", "decay_la") for path in ("segment", "slices")] + \
        [("kda", "f32", 64, "slices"), ("gdn", "f32", 64, "slices"), ("decay_la", "f32", 64, "slices")]


@pytest.mark.parametrize("kind,dt,D,path", CASES, ids=lambda c: str(c))
def test_backward_varlen_matches_oracle_per_sequence(kind, dt, D, path, monkeypatch):
    """Ragged lengths: several chunks with a ragged tail, an empty sequence,
    one token, one short of a chunk, one chunk, one chunk plus one."""
    monkeypatch.setenv("DR_BWD_REV", path)
    dra = _ops()
    lengths = [200, 0, 1, 63, 64, 65, 130, 7]
    x, h0, dhT, do, cu = _packed(kind, dt, D, lengths, seed=41)
    d = to_dev(x)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda:0")
    res = dra.backward_varlen(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], cu_t, h0.to("cuda:0"),
                              do.to("cuda:0"), dhT.to("cuda:0"), flags=flags)
    torch.cuda.synchronize()
    assert (int(flags.item()) & 4) == 0
    got = [None if t is None else t.float().cpu().numpy() for t in res]
    for i in range(len(lengths)):
        a, b = cu[i], cu[i + 1]
        ref = _seq_ref(kind, x, h0, dhT, do, a, b, i)
        _check_seq(got, ref, kind, dt, a, b, i, f"{kind} {dt} D{D}")


@pytest.mark.parametrize("kind", ["kda", "gdn", "decay_la"])
@pytest.mark.parametrize("L", [192, 150])
def test_backward_equal_lengths_match_dense_batch(kind, L, monkeypatch):
    """Packing B sequences of one length reproduces the dense [B, L]
    backward bit for bit, every gradient (same chunks, same arithmetic,
    reductions in a fixed order).  Packed sequences take the value-slice
    reverse pass, so the dense call is pinned to it (DR_BWD_REV=slices); the
    dense default, the segment-parallel pass, is checked against the oracle
    in test_gpu_backward.py."""
    monkeypatch.setenv("DR_BWD_REV", "slices")
    dra = _ops()
    B, H = 3, 4
    w = Workload(f"{kind}_dense_bwd", kind, "bf16", B=B, H=H, T=L, Dk=128, Dv=128, h0_std=0.1, seed=43)
    x = generate(w)
    d = to_dev(x)
    gen = torch.Generator().manual_seed(44)
    do = torch.randn(B, L, H, 128, generator=gen).to(torch.bfloat16).to("cuda:0")
    dhT = (torch.randn(B, H, 128, 128, generator=gen) * 0.1).to("cuda:0")
    r1 = dra.backward(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], do, dhT)
    pk = lambda t: None if t is None else t.reshape(B * L, *t.shape[2:]).contiguous()
    cu = torch.arange(0, B * L + 1, L, dtype=torch.int32, device="cuda:0")
    r2 = dra.backward_varlen(kind, pk(d["q"]), pk(d["k"]), pk(d["v"]), pk(d["g"]), pk(d["beta"]), cu, d["h0"],
                             pk(do), dhT)
    torch.cuda.synchronize()
    names = ["dq", "dk", "dv", "dg", "dbeta"]
    for n, a, b in zip(names, r1[:5], r2[:5]):
        if a is None:
            assert b is None
            continue
        assert torch.equal(pk(a), b), n
    assert torch.equal(r1[5], r2[5]), "dh0"


@pytest.mark.parametrize("kind,dt,D", [("gdn", "bf16", 128), ("kda", "f32", 64), ("decay_la", "bf16", 64)],
                         ids=lambda c: str(c))
def test_backward_varlen_through_prologue(kind, dt, D):
    """Raw projections, ragged lengths: per-sequence gradients against the
    oracle's prologue chain rule on top of its reverse sweep of each
    sequence; dA_log and ddt_bias summed over all sequences."""
    from oracle import prologue as opro
    from delta_rule_rnn_amd.inputs import generate_raw
    dra = _ops()
    lengths = [150, 0, 64, 1, 97]
    T, H, N = sum(lengths), 3, len(lengths)
    w = Workload(f"{kind}_packed_bwd_pro", kind, dt, B=1, H=H, T=T, Dk=D, Dv=D, seed=45)
    x = generate_raw(w)
    gen = torch.Generator().manual_seed(46)
    h0 = torch.randn(N, H, D, D, generator=gen) * 0.2
    dhT = torch.randn(N, H, D, D, generator=gen) * 0.1
    do = torch.randn(1, T, H, D, generator=gen).to(x["q"].dtype)
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    gate = x["A_log"] is not None
    d = to_dev(x)
    delta = kind != "decay_la"
    pro = dra.Prologue(qk_l2norm=True, scale=D ** -0.5, beta_sigmoid=delta, beta_x2=False,
                       A_log=d["A_log"] if gate else None, dt_bias=d["dt_bias"] if gate else None)
    ok = dict(qk_l2norm=True, scale=D ** -0.5, beta_sigmoid=delta, beta_x2=False,
              A_log=x["A_log"] if gate else None, dt_bias=x["dt_bias"] if gate else None)
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda:0")
    res = dra.backward_varlen(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], cu_t, h0.to("cuda:0"),
                              do.to("cuda:0"), dhT.to("cuda:0"), prologue=pro)
    torch.cuda.synchronize()
    got = [None if t is None else t.float().cpu().numpy() for t in res]
    q2, k2, g2, b2 = opro.apply(kind, x["q"], x["k"], x["g"], x["beta"], **ok)
    core_dg = np.zeros_like(g2)
    for i in range(N):
        a, b = cu[i], cu[i + 1]
        sl = lambda t: None if t is None else np.ascontiguousarray(t[:, a:b])
        core = recurrence_backward(kind, sl(q2), sl(k2), x["v"][:, a:b], sl(g2), sl(b2),
                                   h0[i:i + 1].transpose(-1, -2), do[:, a:b], dhT[i:i + 1].transpose(-1, -2))
        core_dg[:, a:b] = core["dg"]
        what = f"{kind} {dt} D{D} seq {i}"
        assert_close_grad(got[5][i:i + 1], np.swapaxes(core["dh0"], -1, -2), dt, f"{what} dh0")
        if b == a:
            continue
        sr = lambda t: None if t is None else t[:, a:b]
        ref = opro.apply_backward(kind, sr(x["q"]), sr(x["k"]), sr(x["g"]), sr(x["beta"]), core["dq"], core["dk"],
                                  core["dg"], core["dbeta"], **ok)
        assert_close_grad(got[0][:, a:b], ref["dq"], dt, f"{what} dq")
        assert_close_grad(got[1][:, a:b], ref["dk"], dt, f"{what} dk")
        assert_close_grad(got[2][:, a:b], core["dv"], dt, f"{what} dv")
        assert_close_grad(got[3][:, a:b], ref["dg"], dt, f"{what} dg")
        if delta:
            assert_close_grad(got[4][:, a:b], ref["dbeta"], dt, f"{what} dbeta")
    if gate:
        # the per-head sums over every token of every sequence, held to the
        # dtype's tolerance times sum_t |coef_t| * max_t |dg^_t|
        tol = 1e-4 if dt == "f32" else 2e-2
        full = opro.apply_backward(kind, x["q"], x["k"], x["g"], x["beta"], np.zeros_like(q2), np.zeros_like(k2),
                                   core_dg, None, **ok)
        gh = opro.scalar_gate(x["g"], x["A_log"], x["dt_bias"])
        coef_dt = -np.exp(opro._f64(x["A_log"])) * opro.sigmoid(opro._f64(x["g"]) + opro._f64(x["dt_bias"]))
        dgmax = np.max(np.abs(core_dg), axis=(0, 1))
        for name, val, coef in (("dA_log", got[6], gh), ("ddt_bias", got[7], coef_dt)):
            scale = np.sum(np.abs(coef), axis=(0, 1)) * dgmax
            err = np.abs(val - full[name])
            assert np.all(err <= tol * scale), f"{kind} {name}: |err| {err} > {tol} * {scale}"
    else:
        assert got[6] is None and got[7] is None


def test_backward_varlen_no_tokens():
    """T = 0 with two (empty) sequences: dh0 = dhT, or zero without dhT."""
    dra = _ops()
    H, D = 2, 64
    z = lambda *s: torch.empty(*s, device="cuda:0")
    q, k, v = z(0, H, D), z(0, H, D), z(0, H, D)
    g, beta, do = z(0, H), z(0, H), z(0, H, D)
    cu = torch.zeros(3, dtype=torch.int32, device="cuda:0")
    dhT = torch.randn(2, H, D, D, device="cuda:0")
    r = dra.backward_varlen("gdn", q, k, v, g, beta, cu, None, do, dhT)
    r0 = dra.backward_varlen("gdn", q, k, v, g, beta, cu, None, do, None)
    torch.cuda.synchronize()
    assert torch.equal(r[5], dhT) and torch.count_nonzero(r0[5]).item() == 0


def test_backward_varlen_bad_offsets_flagged():
    """Offsets that stop short of T (the tail belongs to no sequence): the
    flag is raised, the kernels stay in range, and the sequences the offsets
    do describe still get their own gradients."""
    dra = _ops()
    lengths = [50, 70, 30]
    x, h0, dhT, do, cu = _packed("gdn", "f32", 64, lengths, seed=47, H=2)
    bad = cu[:-1]                     # 2 sequences over [0, 50) and [50, 120); T = 150
    d = to_dev(x)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    cu_t = torch.tensor(bad, dtype=torch.int32, device="cuda:0")
    res = dra.backward_varlen("gdn", d["q"], d["k"], d["v"], d["g"], d["beta"], cu_t, h0[:2].to("cuda:0"),
                              do.to("cuda:0"), dhT[:2].to("cuda:0"), flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) & 4
    got = [None if t is None else t.float().cpu().numpy() for t in res]
    for i in range(2):
        a, b = bad[i], bad[i + 1]
        ref = _seq_ref("gdn", x, h0, dhT, do, a, b, i)
        _check_seq(got, ref, "gdn", "f32", a, b, i, "short offsets")


def test_backward_varlen_full_size_sampled():
    """The packed workload of bench.py --mode varlen (the 32 768 tokens of
    the long KDA workload cut into sequences of seeded lengths in [64, 4096])
    through the backward; every gradient of the shortest and the last
    sequence on one sampled head against the oracle run on each alone."""
    dra = _ops()
    from delta_rule_rnn_amd.inputs import WORKLOADS, packed_lengths
    w = WORKLOADS["kda_bf16_long"]
    lengths = packed_lengths(w.T, seed=7)
    x = generate(w)
    N = len(lengths)
    gen = torch.Generator().manual_seed(48)
    h0 = torch.randn(N, w.H, w.Dk, w.Dv, generator=gen) * 0.1
    dhT = torch.randn(N, w.H, w.Dk, w.Dv, generator=gen) * 0.1
    do = torch.randn(1, w.T, w.H, w.Dv, generator=gen).to(torch.bfloat16)
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    d = to_dev(x)
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda:0")
    res = dra.backward_varlen("kda", d["q"], d["k"], d["v"], d["g"], d["beta"], cu_t, h0.to("cuda:0"),
                              do.to("cuda:0"), dhT.to("cuda:0"))
    torch.cuda.synchronize()
    h = 21
    got = [t[:, :, h:h + 1].float().cpu().numpy() for t in res[:5]]
    dh0 = res[5][:, h:h + 1].cpu().numpy()
    shortest = int(np.argmin(lengths))
    for i in sorted({shortest, N - 1}):
        a, b = cu[i], cu[i + 1]
        sl = lambda t: t[:, a:b, h:h + 1].contiguous()
        ref = recurrence_backward("kda", sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]),
                                  h0[i:i + 1, h:h + 1].transpose(-1, -2), sl(do),
                                  dhT[i:i + 1, h:h + 1].transpose(-1, -2))
        for name, val in zip(["dq", "dk", "dv", "dg", "dbeta"], got):
            assert_close_grad(val[:, a:b], ref[name], "bf16", f"seq {i} (length {b - a}) head {h} {name}")
        assert_close_grad(dh0[i:i + 1], np.swapaxes(ref["dh0"], -1, -2), "bf16", f"seq {i} head {h} dh0")
