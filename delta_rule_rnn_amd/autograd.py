"""Differentiable entry point: the library's forward (dr_forward /
dr_forward_varlen) and its backward (dr_backward_prologue /
dr_backward_varlen) as one torch.autograd.Function, so that the recurrence
can sit inside a model trained with torch.autograd.  Argument marshalling
only: both directions run in the HIP library.

The backward recomputes everything it needs from the saved inputs (the
forward keeps no intermediate), as the chunk-form backward of the page
"Gated DeltaNet" (section "反向传播：状态伴随与三角变换梯度") does.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import ops
from .ops import Prologue


def _prologue(flags, A_log, dt_bias) -> Optional[Prologue]:
    if flags is None:
        return None
    qk, scale, sig, x2 = flags
    return Prologue(qk_l2norm=qk, scale=scale, beta_sigmoid=sig, beta_x2=x2, A_log=A_log, dt_bias=dt_bias)


class _DeltaRule(torch.autograd.Function):
    @staticmethod
    def forward(ctx, kind, q, k, v, g, beta, h0, A_log, dt_bias, cu_seqlens, pro_flags):
        pro = _prologue(pro_flags, A_log, dt_bias)
        if cu_seqlens is None:
            o, hT = ops.forward(kind, q, k, v, g, beta, h0, output_final_state=True, prologue=pro)
        else:
            o, hT = ops.forward_varlen(kind, q, k, v, g, beta, cu_seqlens, h0, output_final_state=True,
                                       prologue=pro)
        ctx.kind = kind
        ctx.pro_flags = pro_flags
        ctx.set_materialize_grads(False)
        ctx.save_for_backward(q, k, v, g, beta, h0, A_log, dt_bias, cu_seqlens)
        ctx.mark_non_differentiable(*([cu_seqlens] if cu_seqlens is not None else []))
        return o, hT

    @staticmethod
    def backward(ctx, do, dhT):
        q, k, v, g, beta, h0, A_log, dt_bias, cu = ctx.saved_tensors
        if do is None:
            do = torch.zeros(*v.shape, dtype=q.dtype, device=q.device)
        do = do.contiguous()
        dhT = None if dhT is None else dhT.contiguous()
        pro = _prologue(ctx.pro_flags, A_log, dt_bias)
        if cu is None:
            res = ops.backward(ctx.kind, q, k, v, g, beta, h0, do, dhT, prologue=pro)
        else:
            res = ops.backward_varlen(ctx.kind, q, k, v, g, beta, cu, h0, do, dhT, prologue=pro)
        dq, dk, dv, dg, dbeta, dh0 = res[:6]
        dA_log, ddt = (res[6], res[7]) if pro is not None else (None, None)
        return (None, dq, dk, dv, dg, dbeta if beta is not None else None, dh0 if h0 is not None else None,
                dA_log if A_log is not None else None, ddt if dt_bias is not None else None, None, None)


def chunk_delta_rule(kind: str, q, k, v, g, beta=None, initial_state=None, output_final_state: bool = False,
                     cu_seqlens=None, prologue: Optional[Prologue] = None
                     ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """The chunkwise gated delta rule of ``kind`` ("kda", "gdn" or
    "decay_la"), differentiable in q, k, v, g, beta, initial_state and the
    prologue's A_log / dt_bias.

    Dense: q, k [B,T,H,Dk], v [B,T,H,Dv]; g [B,T,H,Dk] (kda) or [B,T,H];
    beta [B,T,H] (ignored for decay_la); initial_state fp32 [B,H,Dk,Dv].
    Packed (cu_seqlens int32 [N+1] on the device): the same with a batch of
    one (or none), initial_state [N,H,Dk,Dv].  Returns (o, final_state), the
    final state None unless requested (its gradient flows either way)."""
    if kind == "decay_la":
        beta = None
    flags = None
    A_log = dt_bias = None
    if prologue is not None:
        flags = (bool(prologue.qk_l2norm), float(prologue.scale), bool(prologue.beta_sigmoid),
                 bool(prologue.beta_x2))
        A_log, dt_bias = prologue.A_log, prologue.dt_bias
    o, hT = _DeltaRule.apply(kind, q, k, v, g, beta, initial_state, A_log, dt_bias, cu_seqlens, flags)
    return o, (hT if output_final_state else None)
