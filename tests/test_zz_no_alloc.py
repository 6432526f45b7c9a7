"""dr_forward_noalloc (the forward with the library's static scratch array as
its workspace) against dr_forward with a caller workspace: the same kernels
on the same inputs, so the results must be bit-identical.  Two calls in a
row, the second smaller, so that the second runs over what the first left in
the array; then a problem over the array's limit is refused."""
from __future__ import annotations

import pytest
import torch

from delta_rule_rnn_amd.inputs import WORKLOADS, generate

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run_both(kind, w, prologue=None):
    import delta_rule_rnn_amd as dra
    from delta_rule_rnn_amd import ops
    x = {n: (t.to(DEV) if t is not None else None) for n, t in generate(w).items()}
    beta = None if kind == "decay_la" else x["beta"]
    ws = ops.alloc_workspace(kind, x["q"], x["v"])
    # dr_forward with the caller's workspace (through the prologue entry point
    # so that both calls take the same C entry path)
    pro = prologue or dra.Prologue()
    o_ref, h_ref = ops._forward(kind, x["q"], x["k"], x["v"], x["g"], beta, x["h0"], True, 64, ws, None, None,
                                prologue=pro)
    o, h = dra.forward_noalloc(kind, x["q"], x["k"], x["v"], x["g"], beta, x["h0"], prologue=pro)
    torch.cuda.synchronize()
    return o, h, o_ref, h_ref


@pytest.mark.parametrize("kind,base", [("kda", "kda_bf16"), ("gdn", "gdn_f32_small"), ("decay_la", "la_bf16")])
def test_noalloc_matches_workspace_forward_twice(kind, base):
    # first call: several chunks per chain, ragged tail; second: smaller
    for B, H, T in ((2, 4, 1000), (1, 2, 130)):
        w = WORKLOADS[base].with_(B=B, H=H, T=T, h0_std=0.1, seed=B * 100 + T)
        print(f"noalloc {kind} {base} B={B} H={H} T={T}", flush=True)
        o, h, o_ref, h_ref = _run_both(kind, w)
        assert torch.equal(o, o_ref), f"{kind} B={B} T={T}: o differs"
        assert torch.equal(h, h_ref), f"{kind} B={B} T={T}: hT differs"


def test_noalloc_refuses_problems_over_the_limit():
    import delta_rule_rnn_amd as dra
    from delta_rule_rnn_amd import _lib, ops
    lib = _lib.load()
    cap = lib.dr_noalloc_scratch_bytes()
    T = 64
    while ops.workspace_bytes("kda", 1, T, 8, 128, 128, torch.bfloat16) <= cap:
        T *= 2
    w = WORKLOADS["kda_bf16"].with_(B=1, H=8, T=T, seed=3)
    x = {n: (t.to(DEV) if t is not None else None) for n, t in generate(w).items()}
    with pytest.raises(dra.DeltaRuleError, match="static scratch"):
        dra.forward_noalloc("kda", x["q"], x["k"], x["v"], x["g"], x["beta"])
