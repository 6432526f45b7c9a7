"""GPU parity of the recurrent decode step (kda_decode / gdn_decode /
decay_la_decode, through the C ABI) against the fp64 oracle, which is the
token recurrence itself run from the same initial state.

The decode step computes in fp32, so the state after the call is compared
with the fp32 tolerance (max|gpu - ref| / max|ref| <= 1e-4) for every I/O
dtype; outputs use the dtype's tolerance (bf16 outputs are rounded once).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from delta_rule_rnn_amd.inputs import Workload, generate

from .test_gpu_parity import assert_close, to_dev

pytestmark = pytest.mark.gpu


def _ops():
    import delta_rule_rnn_amd as dra
    return dra


def _oracle(kind, x, state):
    """Oracle outputs (o [B,T,H,Dv], final state [B,H,Dk,Dv]) from state."""
    h0 = state.transpose(-1, -2).contiguous() if state is not None else None
    ro, rs = oracle.recurrence(kind, x["q"], x["k"], x["v"], x["g"], x["beta"], h0)
    return ro, np.swapaxes(rs, -1, -2)


CASES = []
for kind in ("kda", "gdn", "decay_la"):
    for dt in ("f32", "bf16"):
        for D in (64, 128):
            for T in (1, 5):
                CASES.append((kind, dt, D, T))


@pytest.mark.parametrize("kind,dt,D,T", CASES, ids=lambda c: str(c))
def test_decode_matches_oracle(kind, dt, D, T):
    dra = _ops()
    w = Workload(f"{kind}_dec", kind, dt, B=2, H=3, T=T, Dk=D, Dv=D, h0_std=0.5, seed=21)
    x = generate(w)
    d = to_dev(x)
    state = d["h0"].clone()
    o = dra.decode(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], state)
    torch.cuda.synchronize()
    ro, rs = _oracle(kind, x, x["h0"])
    assert_close(o.float().cpu().numpy(), ro, dt, f"{kind} {dt} D{D} T{T} output")
    assert_close(state.cpu().numpy(), rs, "f32", f"{kind} {dt} D{D} T{T} state")


@pytest.mark.parametrize("kind", ["kda", "gdn", "decay_la"])
def test_prefill_then_decode(kind):
    """A chunked prefill's final state continues in the decode step: outputs
    and state match one oracle pass over all tokens."""
    dra = _ops()
    T1, T2 = 200, 7
    w = Workload(f"{kind}_cont", kind, "bf16", B=2, H=4, T=T1 + T2, Dk=128, Dv=128, h0_std=0.1, seed=22)
    x = generate(w)
    d = to_dev(x)
    cut = lambda t, a, b: None if t is None else t[:, a:b].contiguous()
    _, hT = dra.forward(kind, cut(d["q"], 0, T1), cut(d["k"], 0, T1), cut(d["v"], 0, T1),
                        cut(d["g"], 0, T1), cut(d["beta"], 0, T1), d["h0"])
    o2 = dra.decode(kind, cut(d["q"], T1, T1 + T2), cut(d["k"], T1, T1 + T2), cut(d["v"], T1, T1 + T2),
                    cut(d["g"], T1, T1 + T2), cut(d["beta"], T1, T1 + T2), hT)
    torch.cuda.synchronize()
    ro, rs = _oracle(kind, x, x["h0"])
    assert_close(o2.float().cpu().numpy(), ro[:, T1:], "bf16", f"{kind} decode after prefill, output")
    assert_close(hT.cpu().numpy(), rs, "bf16", f"{kind} decode after prefill, state")


def test_decode_no_tokens_keeps_state():
    dra = _ops()
    w = Workload("kda_dec0", "kda", "bf16", B=1, H=2, T=0, Dk=64, Dv=64, h0_std=1.0, seed=23)
    d = to_dev(generate(w))
    state = d["h0"].clone()
    o = dra.kda_decode(d["q"], d["k"], d["v"], d["g"], d["beta"], state)
    torch.cuda.synchronize()
    assert o.shape == (1, 0, 2, 64) and torch.equal(state, d["h0"])


def test_decode_large_batch_sampled():
    """Serving-sized call (64 sequences x 32 heads, one token each), sampled
    chains against the oracle."""
    dra = _ops()
    w = Workload("kda_dec_big", "kda", "bf16", B=64, H=32, T=1, Dk=128, Dv=128, h0_std=0.5, seed=24)
    x = generate(w)
    d = to_dev(x)
    state = d["h0"].clone()
    o = dra.kda_decode(d["q"], d["k"], d["v"], d["g"], d["beta"], state)
    torch.cuda.synchronize()
    o, state = o.float().cpu().numpy(), state.cpu().numpy()
    for (b, h) in [(0, 0), (17, 5), (63, 31), (40, 16)]:
        sl = lambda t: None if t is None else t[b:b + 1, :, h:h + 1].contiguous()
        xs = {n: sl(t) for n, t in x.items() if n != "h0"}
        ro, rs = _oracle("kda", xs, x["h0"][b:b + 1, h:h + 1])
        assert_close(o[b:b + 1, :, h:h + 1], ro, "bf16", f"chain ({b},{h}) output")
        assert_close(state[b:b + 1, h:h + 1], rs, "f32", f"chain ({b},{h}) state")


def test_decode_streaming_stores_sampled():
    """A call whose state (160 x 32 heads x 64 KB = 335 MB) exceeds the
    128 MB threshold above which the state is written back with streaming
    stores; sampled chains against the oracle, two calls in a row."""
    dra = _ops()
    w = Workload("kda_dec_stream", "kda", "bf16", B=160, H=32, T=2, Dk=128, Dv=128, h0_std=0.5, seed=25)
    x = generate(w)
    d = to_dev(x)
    state = d["h0"].clone()
    cut = lambda t, a, b: t[:, a:b].contiguous()
    o1 = dra.kda_decode(cut(d["q"], 0, 1), cut(d["k"], 0, 1), cut(d["v"], 0, 1), cut(d["g"], 0, 1),
                        cut(d["beta"], 0, 1), state)
    o2 = dra.kda_decode(cut(d["q"], 1, 2), cut(d["k"], 1, 2), cut(d["v"], 1, 2), cut(d["g"], 1, 2),
                        cut(d["beta"], 1, 2), state)
    torch.cuda.synchronize()
    o = torch.cat([o1, o2], dim=1).float().cpu().numpy()
    state = state.cpu().numpy()
    for (b, h) in [(0, 0), (97, 13), (159, 31)]:
        sl = lambda t: None if t is None else t[b:b + 1, :, h:h + 1].contiguous()
        xs = {n: sl(t) for n, t in x.items() if n != "h0"}
        ro, rs = _oracle("kda", xs, x["h0"][b:b + 1, h:h + 1])
        assert_close(o[b:b + 1, :, h:h + 1], ro, "bf16", f"chain ({b},{h}) output")
        assert_close(state[b:b + 1, h:h + 1], rs, "f32", f"chain ({b},{h}) state")
