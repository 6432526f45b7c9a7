"""GPU: the workspace-poison debug mode.  With DR_POISON_WORKSPACE=1 every
entry point fills its workspace with NaN (all-ones words) before its
launches, so a kernel that reads workspace the call never wrote would put
NaN into the results.  Each call below runs without and with the poison and
must give bit-identical results (every path here is deterministic): the
record path at C = 64 and 128, the segment-parallel path, packed sequences,
the input prologue, the allocation-free forward, and the backward (dense,
and packed through the prologue with gate generation).
"""
from __future__ import annotations

import pytest
import torch

from delta_rule_rnn_amd.inputs import Workload, generate, generate_raw

from .test_gpu_parity import to_dev

pytestmark = pytest.mark.gpu


def _ops():
    import delta_rule_rnn_amd as dra
    return dra


def _same(run, monkeypatch):
    monkeypatch.delenv("DR_POISON_WORKSPACE", raising=False)
    a = run()
    torch.cuda.synchronize()
    monkeypatch.setenv("DR_POISON_WORKSPACE", "1")
    b = run()
    torch.cuda.synchronize()
    monkeypatch.delenv("DR_POISON_WORKSPACE", raising=False)
    assert len(a) == len(b)
    for i, (x, y) in enumerate(zip(a, b)):
        assert (x is None) == (y is None)
        if x is not None:
            assert bool(torch.isfinite(y.float()).all()), f"result {i}: non-finite with the poisoned workspace"
            assert torch.equal(x, y), f"result {i} differs with the poisoned workspace"


@pytest.mark.parametrize("kind,dt,D,C,path", [
    ("kda", "bf16", 128, 64, "records"), ("kda", "bf16", 128, 64, "segment"), ("gdn", "f32", 64, 64, "segment"),
    ("decay_la", "bf16", 64, 64, "records"), ("kda", "bf16", 128, 128, "records"), ("gdn", "f32", 64, 128, "records"),
])
def test_forward_poisoned_workspace(kind, dt, D, C, path, monkeypatch):
    dra = _ops()
    if path == "segment":
        monkeypatch.setenv("DR_FWD_PATH", "segment")
    else:
        monkeypatch.setenv("DR_FWD_PATH", "records")
    w = Workload(f"poison_{kind}", kind, dt, B=2, H=3, T=300, Dk=D, Dv=D, h0_std=0.1, seed=61)
    d = to_dev(generate(w))
    kw = {} if kind == "decay_la" else {"flags": torch.zeros(1, dtype=torch.int32, device="cuda:0")}
    _same(lambda: dra.forward(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], chunk_size=C, **kw),
          monkeypatch)


def test_varlen_prologue_noalloc_poisoned_workspace(monkeypatch):
    dra = _ops()
    w = Workload("poison_pk", "gdn", "bf16", B=1, H=2, T=230, Dk=64, Dv=64, seed=62)
    raw = to_dev(generate_raw(w))
    cu = torch.tensor([0, 100, 100, 230], dtype=torch.int32, device="cuda:0")
    P = dra.Prologue(qk_l2norm=True, scale=0.5, beta_sigmoid=True, A_log=raw["A_log"], dt_bias=raw["dt_bias"])
    _same(lambda: dra.forward_varlen("gdn", raw["q"], raw["k"], raw["v"], raw["g"], raw["beta"], cu_seqlens=cu,
                                     prologue=P), monkeypatch)
    d = to_dev(generate(w))
    _same(lambda: dra.forward_noalloc("gdn", d["q"], d["k"], d["v"], d["g"], d["beta"]), monkeypatch)


@pytest.mark.parametrize("kind", ["kda", "gdn", "decay_la"])
def test_backward_poisoned_workspace(kind, monkeypatch):
    dra = _ops()
    w = Workload(f"poison_bwd_{kind}", kind, "bf16", B=2, H=2, T=200, Dk=64, Dv=64, h0_std=0.2, seed=63)
    d = to_dev(generate(w))
    gen = torch.Generator().manual_seed(64)
    do = torch.randn(d["v"].shape, generator=gen).to(torch.bfloat16).to("cuda:0")
    dhT = (torch.randn(d["h0"].shape, generator=gen) * 0.1).to("cuda:0")
    _same(lambda: dra.backward(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], do, dhT), monkeypatch)


def test_backward_varlen_prologue_poisoned_workspace(monkeypatch):
    dra = _ops()
    w = Workload("poison_bwd_pk", "gdn", "bf16", B=1, H=2, T=230, Dk=64, Dv=64, seed=65)
    raw = to_dev(generate_raw(w))
    cu = torch.tensor([0, 100, 100, 230], dtype=torch.int32, device="cuda:0")
    P = dra.Prologue(qk_l2norm=True, scale=0.5, beta_sigmoid=True, A_log=raw["A_log"], dt_bias=raw["dt_bias"])
    sq = lambda t: t[0].contiguous()
    do = torch.randn(230, 2, 64, generator=torch.Generator().manual_seed(66)).to(torch.bfloat16).to("cuda:0")
    _same(lambda: dra.backward_varlen("gdn", sq(raw["q"]), sq(raw["k"]), sq(raw["v"]), sq(raw["g"]),
                                      sq(raw["beta"]), cu, None, do, None, prologue=P), monkeypatch)
