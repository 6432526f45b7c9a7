"""GPU parity over seeded random shapes: kind, dtype, head size, batch,
heads, sequence length (ragged, from one token to several chunks), with or
without an initial state; the forward and the backward of the dense layout
and the forward and backward of packed sequences of random lengths (empty
ones included), each against the fp64 oracle.  Tolerances as in
test_gpu_parity (fp32 I/O max-rel 1e-4; bf16 I/O rel-L2 and max-rel 2e-2).
"""
from __future__ import annotations

import random

import numpy as np
import pytest
import torch

import oracle
from oracle.backward import recurrence_backward
from delta_rule_rnn_amd.inputs import Workload, generate

from .test_gpu_parity import assert_close, assert_close_grad, to_dev

pytestmark = pytest.mark.gpu


def _ops():
    import delta_rule_rnn_amd as dra
    return dra


def _shape(seed):
    r = random.Random(seed)
    kind = r.choice(["kda", "gdn", "decay_la"])
    dt = r.choice(["f32", "bf16"])
    D = r.choice([64, 128])
    B, H = r.randint(1, 3), r.randint(1, 4)
    T = r.choice([r.randint(1, 64), r.randint(65, 400)])
    h0 = r.random() < 0.7
    return kind, dt, D, B, H, T, h0


@pytest.mark.parametrize("seed", range(12))
def test_random_dense_forward_backward(seed):
    dra = _ops()
    kind, dt, D, B, H, T, use_h0 = _shape(seed)
    w = Workload(f"rand{seed}", kind, dt, B=B, H=H, T=T, Dk=D, Dv=D, h0_std=0.2 if use_h0 else 0.0,
                 seed=1000 + seed)
    x = generate(w)
    d = to_dev(x)
    what = f"seed {seed}: {kind} {dt} D{D} B{B} H{H} T{T} h0={use_h0}"
    o, hT = dra.forward(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    gen = torch.Generator().manual_seed(2000 + seed)
    do = torch.randn(B, T, H, D, generator=gen).to(x["q"].dtype)
    dhT = torch.randn(B, H, D, D, generator=gen) * 0.1
    res = dra.backward(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], do.to("cuda:0"), dhT.to("cuda:0"))
    torch.cuda.synchronize()
    h0 = None if x["h0"] is None else x["h0"].transpose(-1, -2)
    ro, rs = oracle.recurrence(kind, x["q"], x["k"], x["v"], x["g"], x["beta"], h0)
    assert_close(o.float().cpu().numpy(), ro, dt, f"{what} output")
    assert_close(hT.cpu().numpy(), np.swapaxes(rs, -1, -2), dt, f"{what} state")
    ref = recurrence_backward(kind, x["q"], x["k"], x["v"], x["g"], x["beta"], h0, do, dhT.transpose(-1, -2))
    got = [None if t is None else t.float().cpu().numpy() for t in res]
    for name, val in zip(["dq", "dk", "dv", "dg"], got[:4]):
        assert_close_grad(val, ref[name], dt, f"{what} {name}")
    if kind != "decay_la":
        assert_close_grad(got[4], ref["dbeta"], dt, f"{what} dbeta")
    assert_close_grad(got[5], np.swapaxes(ref["dh0"], -1, -2), dt, f"{what} dh0")


@pytest.mark.parametrize("seed", range(8))
def test_random_packed_forward_backward(seed):
    dra = _ops()
    r = random.Random(500 + seed)
    kind, dt, D, _, H, _, _ = _shape(500 + seed)
    N = r.randint(1, 5)
    lengths = [r.choice([0, r.randint(1, 64), r.randint(65, 200)]) for _ in range(N)]
    if sum(lengths) == 0:
        lengths[0] = 1
    T = sum(lengths)
    w = Workload(f"randpk{seed}", kind, dt, B=1, H=H, T=T, Dk=D, Dv=D, seed=3000 + seed)
    x = generate(w)
    gen = torch.Generator().manual_seed(4000 + seed)
    h0 = torch.randn(N, H, D, D, generator=gen) * 0.2
    dhT = torch.randn(N, H, D, D, generator=gen) * 0.1
    do = torch.randn(1, T, H, D, generator=gen).to(x["q"].dtype)
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    d = to_dev(x)
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda:0")
    o, hT = dra.forward_varlen(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], cu_t, h0=h0.to("cuda:0"))
    res = dra.backward_varlen(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], cu_t, h0.to("cuda:0"),
                              do.to("cuda:0"), dhT.to("cuda:0"))
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    hT = hT.cpu().numpy()
    got = [None if t is None else t.float().cpu().numpy() for t in res]
    what = f"seed {seed}: {kind} {dt} D{D} H{H} lengths {lengths}"
    for i in range(N):
        a, b = cu[i], cu[i + 1]
        sl = lambda t: None if t is None else t[:, a:b].contiguous()
        hi = h0[i:i + 1].transpose(-1, -2)
        ro, rs = oracle.recurrence(kind, sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]),
                                   hi.contiguous())
        assert_close(hT[i:i + 1], np.swapaxes(rs, -1, -2), dt, f"{what} seq {i} state")
        ref = recurrence_backward(kind, sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]), hi,
                                  sl(do), dhT[i:i + 1].transpose(-1, -2))
        assert_close_grad(got[5][i:i + 1], np.swapaxes(ref["dh0"], -1, -2), dt, f"{what} seq {i} dh0")
        if b == a:
            continue
        assert_close(o[:, a:b], ro, dt, f"{what} seq {i} output")
        for name, val in zip(["dq", "dk", "dv", "dg"], got[:4]):
            assert_close_grad(val[:, a:b], ref[name], dt, f"{what} seq {i} {name}")
        if kind != "decay_la":
            assert_close_grad(got[4][:, a:b], ref["dbeta"], dt, f"{what} seq {i} dbeta")


@pytest.mark.parametrize("seed", range(16))
def test_random_forward_path_and_chunk(seed, monkeypatch):
    """The forward over random shapes on a random path (segment-parallel or
    record) and chunk size (64, or 128 where built), long enough for many
    segments (up to 40 chunks per chain, so segments of one or a few
    chunks), against the oracle."""
    dra = _ops()
    r = random.Random(5000 + seed)
    kind = r.choice(["kda", "gdn", "decay_la"])
    dt = r.choice(["f32", "bf16"])
    D = r.choice([64, 128])
    C = r.choice([64, 128]) if (dt == "bf16" or D == 64) else 64
    path = r.choice(["segment", "records"])
    B, H = r.randint(1, 3), r.randint(1, 4)
    T = r.choice([r.randint(1, 130), r.randint(131, 2500)])
    use_h0 = r.random() < 0.7
    monkeypatch.setenv("DR_FWD_PATH", path)
    w = Workload(f"randp{seed}", kind, dt, B=B, H=H, T=T, Dk=D, Dv=D, h0_std=0.2 if use_h0 else 0.0,
                 seed=6000 + seed)
    x = generate(w)
    d = to_dev(x)
    what = f"seed {seed}: {kind} {dt} D{D} C{C} {path} B{B} H{H} T{T} h0={use_h0}"
    print(what, flush=True)
    o, hT = dra.forward(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], chunk_size=C)
    torch.cuda.synchronize()
    h0 = None if x["h0"] is None else x["h0"].transpose(-1, -2)
    ro, rs = oracle.recurrence(kind, x["q"], x["k"], x["v"], x["g"], x["beta"], h0)
    assert_close(o.float().cpu().numpy(), ro, dt, f"{what} output")
    assert_close(hT.cpu().numpy(), np.swapaxes(rs, -1, -2), dt, f"{what} state")
