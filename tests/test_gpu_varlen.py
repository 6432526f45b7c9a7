"""GPU parity of the packed-sequence forward (kda_fwd_varlen / gdn_fwd_varlen
/ decay_la_fwd_varlen, through the C ABI): each sequence against the fp64
oracle run on that sequence alone, packing of equal lengths against the
dense batched forward (bit-identical: same chunks, same arithmetic), and the
flag raised for malformed offsets (which the kernels clamp into range).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from delta_rule_rnn_amd.inputs import Workload, generate

from .test_gpu_parity import assert_close, assert_close_grad, to_dev

pytestmark = pytest.mark.gpu


def _ops():
    import delta_rule_rnn_amd as dra
    return dra


def _packed(kind, dt, D, lengths, seed, H=3):
    """Inputs of len(lengths) sequences drawn as one batch of T = sum tokens,
    plus per-sequence initial states; cu_seqlens as a list."""
    T = int(sum(lengths))
    w = Workload(f"{kind}_packed", kind, dt, B=1, H=H, T=T, Dk=D, Dv=D, seed=seed)
    x = generate(w)
    N = len(lengths)
    h0 = torch.randn(N, H, D, D, generator=torch.Generator().manual_seed(seed + 1)) * 0.2
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return x, h0, cu


CASES = [("kda", "bf16", 128), ("gdn", "bf16", 128), ("decay_la", "bf16", 128),
         ("kda", "f32", 64), ("gdn", "f32", 64), ("decay_la", "f32", 64)]


@pytest.mark.parametrize("kind,dt,D", CASES, ids=lambda c: str(c))
def test_varlen_matches_oracle_per_sequence(kind, dt, D):
    dra = _ops()
    lengths = [200, 0, 1, 63, 64, 65, 130, 7]
    x, h0, cu = _packed(kind, dt, D, lengths, seed=31)
    d = to_dev(x)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda:0")
    o, hT = dra.forward_varlen(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], cu_t, h0=h0.to("cuda:0"),
                               flags=flags)
    torch.cuda.synchronize()
    assert (int(flags.item()) & 4) == 0
    o, hT = o.float().cpu().numpy()[0], hT.cpu().numpy()
    for i, n in enumerate(lengths):
        a, b = cu[i], cu[i + 1]
        sl = lambda t: None if t is None else t[:, a:b].contiguous()
        ro, rs = oracle.recurrence(kind, sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]),
                                   h0[i:i + 1].transpose(-1, -2).contiguous())
        if n > 0:
            assert_close(o[a:b][None], ro, dt, f"{kind} {dt} sequence {i} (length {n}) output")
        assert_close(hT[i:i + 1], np.swapaxes(rs, -1, -2), dt, f"{kind} {dt} sequence {i} (length {n}) state")


@pytest.mark.parametrize("kind", ["kda", "gdn", "decay_la"])
@pytest.mark.parametrize("L", [192, 150])
def test_equal_lengths_match_dense_batch(kind, L, monkeypatch):
    """Packing B sequences of one length reproduces the dense [B, L] forward
    of the record path (the path packed sequences take) bit for bit."""
    monkeypatch.setenv("DR_FWD_PATH", "records")
    dra = _ops()
    B, H = 3, 4
    w = Workload(f"{kind}_dense", kind, "bf16", B=B, H=H, T=L, Dk=128, Dv=128, h0_std=0.1, seed=33)
    d = to_dev(generate(w))
    o1, h1 = dra.forward(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    pk = lambda t: None if t is None else t.reshape(B * L, *t.shape[2:]).contiguous()
    cu = torch.arange(0, B * L + 1, L, dtype=torch.int32, device="cuda:0")
    o2, h2 = dra.forward_varlen(kind, pk(d["q"]), pk(d["k"]), pk(d["v"]), pk(d["g"]), pk(d["beta"]), cu,
                                h0=d["h0"])
    torch.cuda.synchronize()
    assert torch.equal(o2.reshape(B, L, H, 128), o1) and torch.equal(h2, h1)


def test_malformed_offsets_raise_flag():
    """Offsets that decrease or leave [0, T] are clamped by the kernels (every
    access stays inside the tensors) and reported through flag 0x4."""
    dra = _ops()
    x, h0, _ = _packed("gdn", "bf16", 64, [100, 100, 100], seed=35, H=2)
    d = to_dev(x)
    for cu in ([0, 100, 50, 300], [0, 100, 200, 301], [5, 100, 200, 300]):
        flags = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda:0")
        o, hT = dra.forward_varlen("gdn", d["q"], d["k"], d["v"], d["g"], d["beta"], cu_t, flags=flags)
        torch.cuda.synchronize()
        assert int(flags.item()) & 4, cu
        assert torch.isfinite(hT).all()


def test_varlen_full_size_sampled():
    """The packed workload bench.py --mode varlen times: the 32 768 tokens of
    the KDA benchmark workload cut into sequences of seeded lengths in
    [64, 4096]; three sampled sequences on two heads against the oracle run
    on each alone."""
    dra = _ops()
    from delta_rule_rnn_amd.inputs import WORKLOADS
    w0 = WORKLOADS["kda_bf16_long"]
    T = w0.B * w0.T
    w = w0.with_(name=w0.name + "_packed", B=1, T=T)
    rng = torch.Generator().manual_seed(7)
    lengths, left = [], T
    while left > 0:
        n = min(left, int(torch.randint(64, 4097, (1,), generator=rng).item()))
        lengths.append(n)
        left -= n
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    x = generate(w)
    d = to_dev(x)
    sq = lambda t: None if t is None else t[0]
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda:0")
    o, hT = dra.forward_varlen("kda", sq(d["q"]), sq(d["k"]), sq(d["v"]), sq(d["g"]), sq(d["beta"]), cu_t)
    torch.cuda.synchronize()
    o, hT = o.float().cpu().numpy(), hT.cpu().numpy()
    for i in (0, len(lengths) // 2, len(lengths) - 1):
        a, b = cu[i], cu[i + 1]
        for h in (3, 29):
            sl = lambda t: t[:, a:b, h:h + 1].contiguous()
            ro, rs = oracle.recurrence("kda", sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]))
            assert_close(o[a:b, h:h + 1][None], ro, "bf16", f"sequence {i} head {h} output")
            assert_close(hT[i:i + 1, h:h + 1], np.swapaxes(rs, -1, -2), "bf16", f"sequence {i} head {h} state")


def test_many_short_sequences():
    """2500 sequences of lengths 0..20 (the chunk table is built in blocks of
    1024 sequences, with a carry between blocks): sequences on both sides of
    each block boundary, and a spread of others, against the oracle, for
    the forward and the backward."""
    import random
    from oracle.backward import recurrence_backward
    dra = _ops()
    r = random.Random(41)
    lengths = [r.randint(0, 20) for _ in range(2500)]
    x, h0, cu = _packed("gdn", "f32", 64, lengths, seed=42, H=1)
    N, T = len(lengths), cu[-1]
    d = to_dev(x)
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda:0")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    gen = torch.Generator().manual_seed(43)
    do = torch.randn(1, T, 1, 64, generator=gen)
    dhT = torch.randn(N, 1, 64, 64, generator=gen) * 0.1
    o, hT = dra.forward_varlen("gdn", d["q"], d["k"], d["v"], d["g"], d["beta"], cu_t, h0=h0.to("cuda:0"),
                               flags=flags)
    res = dra.backward_varlen("gdn", d["q"], d["k"], d["v"], d["g"], d["beta"], cu_t, h0.to("cuda:0"),
                              do.to("cuda:0"), dhT.to("cuda:0"))
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    o, hT = o.cpu().numpy(), hT.cpu().numpy()
    got = [t.cpu().numpy() for t in res]
    picks = sorted({0, 1, 1022, 1023, 1024, 1025, 2046, 2047, 2048, 2049, N - 1} | set(r.sample(range(N), 20)))
    for i in picks:
        a, b = cu[i], cu[i + 1]
        sl = lambda t: t[:, a:b].contiguous()
        hi = h0[i:i + 1].transpose(-1, -2).contiguous()
        ro, rs = oracle.recurrence("gdn", sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]), hi)
        assert_close(hT[i:i + 1], np.swapaxes(rs, -1, -2), "f32", f"sequence {i} (length {b - a}) state")
        ref = recurrence_backward("gdn", sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]), hi,
                                  sl(do), dhT[i:i + 1].transpose(-1, -2))
        assert_close_grad(got[5][i:i + 1], np.swapaxes(ref["dh0"], -1, -2), "f32", f"sequence {i} dh0")
        if b > a:
            assert_close(o[:, a:b], ro, "f32", f"sequence {i} output")
            for name, val in zip(["dq", "dk", "dv", "dg", "dbeta"], got[:5]):
                assert_close_grad(val[:, a:b], ref[name], "f32", f"sequence {i} {name}")
