"""Thin torch-facing binding over the C ABI (argument marshalling only: every
step of the computation runs in the library's HIP kernels).

Tensors must live on the GPU, be contiguous and use the documented dtypes;
outputs and the workspace are allocated here with torch and handed to the
library as raw pointers, together with torch's current HIP stream.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from . import _lib

DR_F32, DR_BF16 = 0, 1
KINDS = {"kda": 0, "gdn": 1, "decay_la": 2}
CHUNK = 64


class DeltaRuleError(RuntimeError):
    pass


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = _lib.load().dr_status_string(status).decode()
        raise DeltaRuleError(f"{what} failed: {msg} (status {status})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DR_BF16
    if t.dtype == torch.float32:
        return DR_F32
    raise DeltaRuleError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t: Optional[torch.Tensor], name: str, dtype=None, shape=None):
    if t is None:
        return
    if not t.is_cuda:
        raise DeltaRuleError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise DeltaRuleError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise DeltaRuleError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise DeltaRuleError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


@dataclass
class Prologue:
    """Input prologue applied inside the kernels (struct dr_prologue):
    q, k L2-normalised per token and head (eps 1e-6) when ``qk_l2norm``, then
    q scaled by ``scale``; beta through a sigmoid (doubled with ``beta_x2``);
    and, when ``A_log`` is given (scalar gates only), the gate input taken as
    the raw projection a: g = -exp(A_log[h]) * softplus(a + dt_bias[h]).
    A_log and dt_bias are fp32 [H] tensors on the GPU."""
    qk_l2norm: bool = False
    scale: float = 1.0
    beta_sigmoid: bool = False
    beta_x2: bool = False
    A_log: Optional[torch.Tensor] = None
    dt_bias: Optional[torch.Tensor] = None

    def to_c(self, H: int) -> _lib.DrPrologue:
        ops = ((_lib.PRO_QK_L2NORM if self.qk_l2norm else 0) | (_lib.PRO_BETA_SIGMOID if self.beta_sigmoid else 0)
               | (_lib.PRO_BETA_X2 if self.beta_x2 else 0) | (_lib.PRO_GATE if self.A_log is not None else 0))
        _need(self.A_log, "A_log", torch.float32, (H,))
        _need(self.dt_bias, "dt_bias", torch.float32, (H,))
        if self.dt_bias is not None and self.A_log is None:
            raise DeltaRuleError("dt_bias without A_log")
        return _lib.DrPrologue(ops, float(self.scale), _ptr(self.A_log), _ptr(self.dt_bias))


def _pro_arg(prologue: Optional[Prologue], H: int):
    """(struct to keep alive, pointer argument) for a prologue or None."""
    if prologue is None:
        return None, None
    c = prologue.to_c(H)
    return c, ctypes.addressof(c)


def workspace_bytes(kind: str, B: int, T: int, H: int, Dk: int, Dv: int, dtype: torch.dtype,
                    chunk_size: int = CHUNK) -> int:
    code = DR_BF16 if dtype == torch.bfloat16 else DR_F32
    return int(_lib.load().dr_workspace_bytes(KINDS[kind], B, T, H, Dk, Dv, chunk_size, code))


def record_bytes(Dk: int, Dv: int, dtype: torch.dtype, chunk_size: int = CHUNK) -> int:
    code = DR_BF16 if dtype == torch.bfloat16 else DR_F32
    return int(_lib.load().dr_record_bytes(Dk, Dv, chunk_size, code))


def record_workspace_bytes(kind: str, B: int, T: int, H: int, Dk: int, Dv: int, dtype: torch.dtype,
                           chunk_size: int = CHUNK) -> int:
    code = DR_BF16 if dtype == torch.bfloat16 else DR_F32
    return int(_lib.load().dr_record_workspace_bytes(KINDS[kind], B, T, H, Dk, Dv, chunk_size, code))


def alloc_workspace(kind, q: torch.Tensor, v: torch.Tensor, chunk_size: int = CHUNK) -> torch.Tensor:
    """Workspace of the full forward entry points (dr_workspace_bytes)."""
    B, T, H, Dk = q.shape
    n = workspace_bytes(kind, B, T, H, Dk, v.shape[-1], q.dtype, chunk_size)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)


def alloc_segment_workspace(kind, q: torch.Tensor, v: torch.Tensor, chunk_size: int = CHUNK) -> torch.Tensor:
    """Workspace of the segment-parallel forward's stages (dr_forward_stage)."""
    B, T, H, Dk = q.shape
    code = DR_BF16 if q.dtype == torch.bfloat16 else DR_F32
    n = int(_lib.load().dr_segment_workspace_bytes(KINDS[kind], B, T, H, Dk, v.shape[-1], chunk_size, code))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)


def alloc_record_workspace(kind, q: torch.Tensor, v: torch.Tensor, chunk_size: int = CHUNK) -> torch.Tensor:
    """Workspace of the record path's step entry points dr_intra / dr_inter."""
    B, T, H, Dk = q.shape
    n = record_workspace_bytes(kind, B, T, H, Dk, v.shape[-1], q.dtype, chunk_size)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)


def _forward(kind: str, q, k, v, g, beta, h0, output_final_state, chunk_size, workspace, flags,
             stream, prologue=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    lib = _lib.load()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    _need(q, "q"); _need(k, "k", dt, q.shape); _need(v, "v", dt, (B, T, H, Dv))
    gshape = (B, T, H, Dk) if kind == "kda" else (B, T, H)
    _need(g, "g", torch.float32, gshape)
    if kind != "decay_la":
        if beta is None:
            raise DeltaRuleError("beta is required")
        _need(beta, "beta", torch.float32, (B, T, H))
    _need(h0, "h0", torch.float32, (B, H, Dk, Dv))
    o = torch.empty(B, T, H, Dv, dtype=dt, device=q.device)
    hT = torch.empty(B, H, Dk, Dv, dtype=torch.float32, device=q.device) if output_final_state else None
    if workspace is None:
        workspace = alloc_workspace(kind, q, v, chunk_size)
    _need(workspace, "workspace", torch.uint8)
    if flags is not None:
        _need(flags, "flags", torch.int32, (1,))
    code = _dtype_code(q)
    common = (B, T, H, Dk, Dv, chunk_size, code, _ptr(workspace), workspace.numel())
    s = _stream(stream)
    if prologue is not None:
        keep, pro = _pro_arg(prologue, H)
        st = lib.dr_forward(KINDS[kind], _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o),
                            _ptr(hT), B, T, H, Dk, Dv, chunk_size, code, pro, _ptr(workspace), workspace.numel(),
                            _ptr(flags), s)
        del keep
        _check(st, "dr_forward")
        return o, hT
    if kind == "kda":
        st = lib.kda_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT),
                         *common, _ptr(flags), s)
    elif kind == "gdn":
        st = lib.gdn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT),
                         *common, _ptr(flags), s)
    else:
        st = lib.decay_la_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h0), _ptr(o), _ptr(hT), *common, s)
    _check(st, f"{kind}_fwd")
    return o, hT


def forward_noalloc(kind: str, q, k, v, g, beta=None, h0=None, output_final_state=True, chunk_size=CHUNK,
                    flags=None, stream=None, prologue: Optional[Prologue] = None):
    """The forward of ``kind`` through dr_forward_noalloc: the library's own
    static device array serves as the workspace (no workspace is allocated
    for the call; o and hT are still allocated here, as for every entry
    point).  Same arguments and results as :func:`forward`."""
    lib = _lib.load()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    _need(q, "q"); _need(k, "k", dt, q.shape); _need(v, "v", dt, (B, T, H, Dv))
    _need(g, "g", torch.float32, (B, T, H, Dk) if kind == "kda" else (B, T, H))
    if kind != "decay_la":
        if beta is None:
            raise DeltaRuleError("beta is required")
        _need(beta, "beta", torch.float32, (B, T, H))
    _need(h0, "h0", torch.float32, (B, H, Dk, Dv))
    if flags is not None:
        _need(flags, "flags", torch.int32, (1,))
    o = torch.empty(B, T, H, Dv, dtype=dt, device=q.device)
    hT = torch.empty(B, H, Dk, Dv, dtype=torch.float32, device=q.device) if output_final_state else None
    keep, pro = _pro_arg(prologue, H)
    st = lib.dr_forward_noalloc(KINDS[kind], _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                _ptr(beta) if kind != "decay_la" else None, _ptr(h0), _ptr(o), _ptr(hT), B, T, H,
                                Dk, Dv, chunk_size, _dtype_code(q), pro, _ptr(flags), _stream(stream))
    del keep
    _check(st, "dr_forward_noalloc")
    return o, hT


def forward_stage(stage: int, kind: str, q, k, v, g, beta=None, h0=None, out=None, hT=None, workspace=None,
                  chunk_size=CHUNK, flags=None, stream=None, prologue: Optional[Prologue] = None) -> None:
    """One stage of the segment-parallel forward (dr_forward_stage): 0 the
    local segment pass (writes out and the workspace), 1 the entry-state
    composition (writes hT), 2 the output correction (updates out).  The
    three in order with one workspace equal :func:`forward`."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    keep, pro = _pro_arg(prologue, H)
    st = _lib.load().dr_forward_stage(stage, KINDS[kind], _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                      _ptr(beta) if kind != "decay_la" else None, _ptr(h0), _ptr(out), _ptr(hT),
                                      B, T, H, Dk, Dv, chunk_size, _dtype_code(q), pro, _ptr(workspace),
                                      0 if workspace is None else workspace.numel(), _ptr(flags), _stream(stream))
    del keep
    _check(st, f"dr_forward_stage({stage})")


def kda_fwd(q, k, v, g, beta, h0=None, output_final_state=True, chunk_size=CHUNK, workspace=None,
            flags=None, stream=None, prologue: Optional[Prologue] = None):
    """KDA forward.  q, k [B,T,H,Dk], v [B,T,H,Dv] (bf16 or fp32); g [B,T,H,Dk]
    fp32 (ln a); beta [B,T,H] fp32; h0 [B,H,Dk,Dv] fp32 or None.
    Returns (o [B,T,H,Dv], hT [B,H,Dk,Dv] fp32 or None)."""
    return _forward("kda", q, k, v, g, beta, h0, output_final_state, chunk_size, workspace, flags, stream,
                    prologue)


def gdn_fwd(q, k, v, g, beta, h0=None, output_final_state=True, chunk_size=CHUNK, workspace=None,
            flags=None, stream=None, prologue: Optional[Prologue] = None):
    """Gated DeltaNet forward: as kda_fwd with g [B,T,H]."""
    return _forward("gdn", q, k, v, g, beta, h0, output_final_state, chunk_size, workspace, flags, stream,
                    prologue)


def decay_la_fwd(q, k, v, g, h0=None, output_final_state=True, chunk_size=CHUNK, workspace=None,
                 stream=None, prologue: Optional[Prologue] = None):
    """Scalar-decay linear attention (no delta term): g [B,T,H], no beta."""
    return _forward("decay_la", q, k, v, g, None, h0, output_final_state, chunk_size, workspace, None,
                    stream, prologue)


FORWARDS = {"kda": kda_fwd, "gdn": gdn_fwd, "decay_la": decay_la_fwd}


def forward(kind: str, q, k, v, g, beta=None, h0=None, **kw):
    if kind == "decay_la":
        return decay_la_fwd(q, k, v, g, h0, **kw)
    return FORWARDS[kind](q, k, v, g, beta, h0, **kw)


# ---- packed sequences -----------------------------------------------------------

def workspace_bytes_varlen(kind: str, N: int, T: int, H: int, Dk: int, Dv: int, dtype: torch.dtype,
                           chunk_size: int = CHUNK) -> int:
    code = DR_BF16 if dtype == torch.bfloat16 else DR_F32
    return int(_lib.load().dr_workspace_bytes_varlen(KINDS[kind], N, T, H, Dk, Dv, chunk_size, code))


def _forward_varlen(kind, q, k, v, g, beta, cu_seqlens, h0, output_final_state, chunk_size, workspace,
                    flags, stream, prologue=None):
    lib = _lib.load()
    squeeze = q.dim() == 4
    if squeeze:
        if q.shape[0] != 1:
            raise DeltaRuleError("packed sequences take q as [T,H,D] or [1,T,H,D]")
        q, k, v = q[0], k[0], v[0]
        g = g[0]
        beta = None if beta is None else beta[0]
    T, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    _need(q, "q"); _need(k, "k", dt, q.shape); _need(v, "v", dt, (T, H, Dv))
    _need(g, "g", torch.float32, (T, H, Dk) if kind == "kda" else (T, H))
    if kind != "decay_la":
        if beta is None:
            raise DeltaRuleError("beta is required")
        _need(beta, "beta", torch.float32, (T, H))
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise DeltaRuleError("cu_seqlens must be int32 [N+1] with N >= 1")
    N = cu_seqlens.numel() - 1
    _need(h0, "h0", torch.float32, (N, H, Dk, Dv))
    o = torch.empty(T, H, Dv, dtype=dt, device=q.device)
    hT = torch.empty(N, H, Dk, Dv, dtype=torch.float32, device=q.device) if output_final_state else None
    need = workspace_bytes_varlen(kind, N, T, H, Dk, Dv, dt, chunk_size)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    if flags is not None:
        _need(flags, "flags", torch.int32, (1,))
    code, s = _dtype_code(q), _stream(stream)
    if prologue is not None:
        keep, pro = _pro_arg(prologue, H)
        st = lib.dr_forward_varlen(KINDS[kind], _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                   N, _ptr(h0), _ptr(o), _ptr(hT), T, H, Dk, Dv, chunk_size, code, pro,
                                   _ptr(workspace), workspace.numel(), _ptr(flags), s)
        del keep
        _check(st, "dr_forward_varlen")
        return (o[None] if squeeze else o), hT
    common = (N, _ptr(h0), _ptr(o), _ptr(hT), T, H, Dk, Dv, chunk_size, code, _ptr(workspace),
              workspace.numel(), _ptr(flags), s)
    if kind == "kda":
        st = lib.kda_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), *common)
    elif kind == "gdn":
        st = lib.gdn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), *common)
    else:
        st = lib.decay_la_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(cu_seqlens), *common)
    _check(st, f"{kind}_fwd_varlen")
    return (o[None] if squeeze else o), hT


def forward_varlen(kind: str, q, k, v, g, beta=None, cu_seqlens=None, h0=None, output_final_state=True,
                   chunk_size=CHUNK, workspace=None, flags=None, stream=None,
                   prologue: Optional[Prologue] = None):
    """Forward over sequences packed along the token axis.  q, k [T,H,Dk]
    (or [1,T,H,Dk]), v [T,H,Dv]; g [T,H,Dk] (kda) or [T,H]; beta [T,H];
    cu_seqlens int32 [N+1] on the device; h0 [N,H,Dk,Dv] or None.
    Returns (o like q with Dv, hT [N,H,Dk,Dv] or None)."""
    if cu_seqlens is None:
        raise DeltaRuleError("cu_seqlens is required")
    return _forward_varlen(kind, q, k, v, g, beta, cu_seqlens, h0, output_final_state, chunk_size,
                           workspace, flags, stream, prologue)


# ---- recurrent decode step ---------------------------------------------------

def _decode(kind: str, q, k, v, g, beta, state, out, stream, prologue=None) -> torch.Tensor:
    lib = _lib.load()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    _need(q, "q"); _need(k, "k", dt, q.shape); _need(v, "v", dt, (B, T, H, Dv))
    _need(g, "g", torch.float32, (B, T, H, Dk) if kind == "kda" else (B, T, H))
    if kind != "decay_la":
        if beta is None:
            raise DeltaRuleError("beta is required")
        _need(beta, "beta", torch.float32, (B, T, H))
    if state is None:
        raise DeltaRuleError("state is required (fp32 [B,H,Dk,Dv], updated in place)")
    _need(state, "state", torch.float32, (B, H, Dk, Dv))
    o = torch.empty(B, T, H, Dv, dtype=dt, device=q.device) if out is None else out
    _need(o, "out", dt, (B, T, H, Dv))
    code, s = _dtype_code(q), _stream(stream)
    if prologue is not None:
        keep, pro = _pro_arg(prologue, H)
        st = lib.dr_decode(KINDS[kind], _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o),
                           B, T, H, Dk, Dv, code, pro, s)
        del keep
        _check(st, "dr_decode")
        return o
    if kind == "kda":
        st = lib.kda_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o),
                            B, T, H, Dk, Dv, code, s)
    elif kind == "gdn":
        st = lib.gdn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o),
                            B, T, H, Dk, Dv, code, s)
    else:
        st = lib.decay_la_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(state), _ptr(o),
                                 B, T, H, Dk, Dv, code, s)
    _check(st, f"{kind}_decode")
    return o


def kda_decode(q, k, v, g, beta, state, out=None, stream=None, prologue: Optional[Prologue] = None) -> torch.Tensor:
    """Apply T new tokens per (b, h) to ``state`` (fp32 [B,H,Dk,Dv], updated
    in place; the layout of a forward's hT) and return o [B,T,H,Dv]."""
    return _decode("kda", q, k, v, g, beta, state, out, stream, prologue)


def gdn_decode(q, k, v, g, beta, state, out=None, stream=None, prologue: Optional[Prologue] = None) -> torch.Tensor:
    """As kda_decode with g [B,T,H]."""
    return _decode("gdn", q, k, v, g, beta, state, out, stream, prologue)


def decay_la_decode(q, k, v, g, state, out=None, stream=None, prologue: Optional[Prologue] = None) -> torch.Tensor:
    """As gdn_decode without beta (no delta term)."""
    return _decode("decay_la", q, k, v, g, None, state, out, stream, prologue)


def decode(kind: str, q, k, v, g, beta=None, state=None, **kw) -> torch.Tensor:
    if kind == "decay_la":
        return decay_la_decode(q, k, v, g, state, **kw)
    return {"kda": kda_decode, "gdn": gdn_decode}[kind](q, k, v, g, beta, state, **kw)


# ---- backward -------------------------------------------------------------------

def backward_workspace_bytes(kind: str, B: int, T: int, H: int, Dk: int, Dv: int, dtype: torch.dtype,
                             chunk_size: int = CHUNK) -> int:
    code = DR_BF16 if dtype == torch.bfloat16 else DR_F32
    return int(_lib.load().dr_backward_workspace_bytes(KINDS[kind], B, T, H, Dk, Dv, chunk_size, code))


def backward(kind: str, q, k, v, g, beta=None, h0=None, do=None, dhT=None, chunk_size=CHUNK, workspace=None,
             stream=None, prologue: Optional[Prologue] = None):
    """Gradients of the forward of ``kind`` given do (the adjoint of o, like
    o) and dhT (the adjoint of hT, fp32 [B,H,Dk,Dv] or None).  Returns
    (dq, dk, dv, dg, dbeta, dh0): dq, dk, dv in the I/O dtype, dg like g,
    dbeta [B,T,H] fp32 (None for decay_la), dh0 fp32 [B,H,Dk,Dv] (zeros
    of h0's shape also when h0 is None).

    With a ``prologue`` (the one the forward took), q, k, g and beta are the
    raw inputs, the gradients are with respect to them, and two more results
    follow: (..., dA_log, ddt_bias), fp32 [H] each (None without gate
    generation, ddt_bias None without dt_bias)."""
    lib = _lib.load()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    _need(q, "q"); _need(k, "k", dt, q.shape); _need(v, "v", dt, (B, T, H, Dv))
    _need(g, "g", torch.float32, (B, T, H, Dk) if kind == "kda" else (B, T, H))
    if kind != "decay_la":
        if beta is None:
            raise DeltaRuleError("beta is required")
        _need(beta, "beta", torch.float32, (B, T, H))
    else:
        beta = None
    if do is None:
        raise DeltaRuleError("do (the adjoint of o) is required")
    _need(do, "do", dt, (B, T, H, Dv))
    _need(h0, "h0", torch.float32, (B, H, Dk, Dv))
    _need(dhT, "dhT", torch.float32, (B, H, Dk, Dv))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty_like(g)
    dbeta = torch.empty_like(beta) if beta is not None else None
    dh0 = torch.empty(B, H, Dk, Dv, dtype=torch.float32, device=q.device)
    code = DR_BF16 if dt == torch.bfloat16 else DR_F32
    if prologue is not None:
        need = int(lib.dr_backward_prologue_workspace_bytes(KINDS[kind], B, T, H, Dk, Dv, chunk_size, code))
    else:
        need = backward_workspace_bytes(kind, B, T, H, Dk, Dv, dt, chunk_size)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    if prologue is None:
        st = lib.dr_backward(KINDS[kind], _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(do),
                             _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0), B, T, H, Dk,
                             Dv, chunk_size, code, _ptr(workspace), workspace.numel(), _stream(stream))
        _check(st, "dr_backward")
        return dq, dk, dv, dg, dbeta, dh0
    gate = prologue.A_log is not None
    dA_log = torch.empty(H, dtype=torch.float32, device=q.device) if gate else None
    ddt = torch.empty(H, dtype=torch.float32, device=q.device) if gate and prologue.dt_bias is not None else None
    keep, pro = _pro_arg(prologue, H)
    st = lib.dr_backward_prologue(KINDS[kind], _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(do),
                                  _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0),
                                  _ptr(dA_log), _ptr(ddt), B, T, H, Dk, Dv, chunk_size, code, pro, _ptr(workspace),
                                  workspace.numel(), _stream(stream))
    del keep
    _check(st, "dr_backward_prologue")
    return dq, dk, dv, dg, dbeta, dh0, dA_log, ddt


def backward_varlen_workspace_bytes(kind: str, N: int, T: int, H: int, Dk: int, Dv: int, dtype: torch.dtype,
                                    chunk_size: int = CHUNK, with_prologue: bool = False) -> int:
    code = DR_BF16 if dtype == torch.bfloat16 else DR_F32
    return int(_lib.load().dr_backward_varlen_workspace_bytes(KINDS[kind], N, T, H, Dk, Dv, chunk_size, code,
                                                              int(with_prologue)))


def backward_varlen(kind: str, q, k, v, g, beta=None, cu_seqlens=None, h0=None, do=None, dhT=None,
                    chunk_size=CHUNK, workspace=None, flags=None, stream=None,
                    prologue: Optional[Prologue] = None):
    """Backward of forward_varlen: sequences packed along the token axis,
    q, k [T,H,Dk] (or [1,T,H,Dk]), v and do [T,H,Dv], g [T,H,Dk] (kda) or
    [T,H], beta [T,H], cu_seqlens int32 [N+1] on the device, h0 and dhT
    [N,H,Dk,Dv] fp32 or None.  Returns what backward() returns, the token
    tensors with the leading 1 kept when q has it and dh0 [N,H,Dk,Dv]."""
    lib = _lib.load()
    if cu_seqlens is None:
        raise DeltaRuleError("cu_seqlens is required")
    squeeze = q.dim() == 4
    if squeeze:
        if q.shape[0] != 1:
            raise DeltaRuleError("packed sequences take q as [T,H,D] or [1,T,H,D]")
        q, k, v, g = q[0], k[0], v[0], g[0]
        beta = None if beta is None else beta[0]
        do = None if do is None else do[0]
    T, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    _need(q, "q"); _need(k, "k", dt, q.shape); _need(v, "v", dt, (T, H, Dv))
    _need(g, "g", torch.float32, (T, H, Dk) if kind == "kda" else (T, H))
    if kind != "decay_la":
        if beta is None:
            raise DeltaRuleError("beta is required")
        _need(beta, "beta", torch.float32, (T, H))
    else:
        beta = None
    if do is None:
        raise DeltaRuleError("do (the adjoint of o) is required")
    _need(do, "do", dt, (T, H, Dv))
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise DeltaRuleError("cu_seqlens must be int32 [N+1] with N >= 1")
    N = cu_seqlens.numel() - 1
    _need(h0, "h0", torch.float32, (N, H, Dk, Dv))
    _need(dhT, "dhT", torch.float32, (N, H, Dk, Dv))
    if flags is not None:
        _need(flags, "flags", torch.int32, (1,))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty_like(g)
    dbeta = torch.empty_like(beta) if beta is not None else None
    dh0 = torch.empty(N, H, Dk, Dv, dtype=torch.float32, device=q.device)
    code = DR_BF16 if dt == torch.bfloat16 else DR_F32
    need = backward_varlen_workspace_bytes(kind, N, T, H, Dk, Dv, dt, chunk_size, prologue is not None)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    gate = prologue is not None and prologue.A_log is not None
    dA_log = torch.empty(H, dtype=torch.float32, device=q.device) if gate else None
    ddt = torch.empty(H, dtype=torch.float32, device=q.device) if gate and prologue.dt_bias is not None else None
    keep, pro = _pro_arg(prologue, H)
    st = lib.dr_backward_varlen(KINDS[kind], _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N,
                                _ptr(h0), _ptr(do), _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta),
                                _ptr(dh0), _ptr(dA_log), _ptr(ddt), T, H, Dk, Dv, chunk_size, code, pro,
                                _ptr(workspace), workspace.numel(), _ptr(flags), _stream(stream))
    del keep
    _check(st, "dr_backward_varlen")
    if squeeze:
        dq, dk, dv, dg = dq[None], dk[None], dv[None], dg[None]
        dbeta = None if dbeta is None else dbeta[None]
    if prologue is None:
        return dq, dk, dv, dg, dbeta, dh0
    return dq, dk, dv, dg, dbeta, dh0, dA_log, ddt


# ---- individual steps ------------------------------------------------------

def chunk_cumsum(g: torch.Tensor, chunk_size: int = CHUNK, stream=None) -> torch.Tensor:
    """Step a1: chunk-local inclusive cumsum of g along T, in log2 units.
    g: [B,T,H,D] or [B,T,H] fp32."""
    _need(g, "g", torch.float32)
    B, T, H = g.shape[:3]
    D = g.shape[3] if g.dim() == 4 else 1
    out = torch.empty_like(g)
    _check(_lib.load().dr_chunk_cumsum(_ptr(g), _ptr(out), B, T, H, D, chunk_size, _stream(stream)),
           "dr_chunk_cumsum")
    return out


def kda_prep(q, k, gamma, chunk_size: int = CHUNK, flags=None, stream=None):
    """Step a2: (qp, kp, km, kbar, phi) from q, k and gamma (step a1 output)."""
    _need(q, "q"); _need(k, "k", q.dtype, q.shape); _need(gamma, "gamma", torch.float32, q.shape)
    B, T, H, Dk = q.shape
    NT = (T + chunk_size - 1) // chunk_size
    qp, kp, km, kbar = (torch.empty_like(q) for _ in range(4))
    phi = torch.empty(B, NT, H, Dk, dtype=torch.float32, device=q.device)
    _check(_lib.load().dr_kda_prep(_ptr(q), _ptr(k), _ptr(gamma), _ptr(qp), _ptr(kp), _ptr(km), _ptr(kbar),
                                   _ptr(phi), B, T, H, Dk, chunk_size, _dtype_code(q), _ptr(flags),
                                   _stream(stream)), "dr_kda_prep")
    return qp, kp, km, kbar, phi


def intra(kind: str, q, k, v, g, beta=None, chunk_size: int = CHUNK, workspace=None, flags=None,
          stream=None) -> torch.Tensor:
    """K1 (steps a1-a3 fused): fills and returns the chunk-record workspace."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if workspace is None:
        workspace = alloc_record_workspace(kind, q, v, chunk_size)
    _check(_lib.load().dr_intra(KINDS[kind], _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), B, T, H, Dk,
                                Dv, chunk_size, _dtype_code(q), _ptr(workspace), workspace.numel(),
                                _ptr(flags), _stream(stream)), "dr_intra")
    return workspace


def inter(kind: str, workspace, B, T, H, Dk, Dv, dtype, h0=None, out=None, hT=None,
          chunk_size: int = CHUNK, stream=None):
    """K2 (steps a4-a5 fused): state pass + output from a filled workspace."""
    dev = workspace.device
    if out is None:
        out = torch.empty(B, T, H, Dv, dtype=dtype, device=dev)
    code = DR_BF16 if dtype == torch.bfloat16 else DR_F32
    _check(_lib.load().dr_inter(KINDS[kind], _ptr(h0), _ptr(out), _ptr(hT), B, T, H, Dk, Dv, chunk_size,
                                code, _ptr(workspace), workspace.numel(), _stream(stream)), "dr_inter")
    return out, hT


def _prow(half, r):
    return 8 * (r >> 2) + 4 * half + (r & 3)


def _pw(w, r):
    return 32 * (w >> 1) + _prow(w & 1, r)


def _frag_maps(C: int, Dk: int, Dv: int):
    """For each record block, the natural (row, col) of every stored element,
    in storage order (the fragment order of include/deltarule.h, dr_intra;
    nw = C/16 position groups, kq = C/32 position blocks)."""
    import numpy as np
    nkb, nw, kq = Dk // 32, C // 16, C // 32
    w, kb, l, j = np.meshgrid(np.arange(nw), np.arange(nkb), np.arange(64), np.arange(8), indexing="ij")
    wq = (_pw(w, l % 16), 32 * kb + 8 * (l // 16) + j)                      # W, Qt: [pos][dk]
    w2, h, kb2, l2, j2 = np.meshgrid(np.arange(nkb), np.arange(2), np.arange(kq), np.arange(64),
                                     np.arange(8), indexing="ij")
    kbt = (32 * w2 + _prow(h, l2 % 16), 32 * kb2 + 8 * (l2 // 16) + j2)     # KbT: [dk][pos]
    w3, kb3, l3, j3 = np.meshgrid(np.arange(nw), np.arange(kq), np.arange(64), np.arange(8), indexing="ij")
    aqk = (_pw(w3, l3 % 16), 32 * kb3 + 8 * (l3 // 16) + j3)                # Aqk: [pos][pos]
    t4, w4, l4, i4 = np.meshgrid(np.arange(Dv // 16), np.arange(nw), np.arange(64), np.arange(4),
                                 indexing="ij")
    ut = (16 * t4 + l4 % 16, 32 * (w4 >> 1) + 8 * (l4 // 16) + 4 * (w4 & 1) + i4)  # UT: [dv][pos]
    return {"W": wq, "Qt": wq, "KbT": kbt, "Aqk": aqk, "UT": ut}


def unpack_records(workspace: torch.Tensor, B: int, T: int, H: int, Dk: int, Dv: int,
                   dtype: torch.dtype, chunk_size: int = CHUNK) -> dict:
    """View the K1 records as natural named tensors: W [B,H,NT,C,Dk],
    Qt [..,C,Dk], KbT [..,Dk,C], Aqk [..,C,C], UT [..,Dv,C], phi [..,Dk]
    (fp32).  The records store each block in the state pass's fragment order
    (include/deltarule.h, dr_intra); this undoes that permutation."""
    import numpy as np
    C = chunk_size
    NT = (T + C - 1) // C
    rb = record_bytes(Dk, Dv, dtype, C)
    esz = torch.tensor([], dtype=dtype).element_size()
    recs = workspace[: B * H * NT * rb].view(B, H, NT, rb)
    maps = _frag_maps(C, Dk, Dv)
    sizes = [("W", C * Dk, (C, Dk)), ("Qt", C * Dk, (C, Dk)), ("KbT", Dk * C, (Dk, C)),
             ("Aqk", C * C, (C, C)), ("UT", Dv * C, (Dv, C))]
    out, off = {}, 0
    for name, n, shp in sizes:
        flat = recs[..., off * esz:(off + n) * esz].contiguous().view(dtype).view(B, H, NT, n)
        rows, cols = (np.asarray(a).reshape(-1) for a in maps[name])
        lin = torch.as_tensor(rows * shp[1] + cols, device=flat.device)
        nat = torch.empty(B, H, NT, n, dtype=dtype, device=flat.device)
        nat[..., lin] = flat
        out[name] = nat.view(B, H, NT, *shp)
        off += n
    pb = off * esz
    out["phi"] = recs[..., pb:pb + Dk * 4].contiguous().view(torch.float32).view(B, H, NT, Dk)
    return out
