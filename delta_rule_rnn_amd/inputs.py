"""Seeded synthetic inputs for the five workloads (shared by tests, the
benchmark and the oracle side of parity checks).

This module holds no arithmetic of the method itself: it only draws random
tensors with the shapes and distributions of the workloads and casts them to
the I/O dtype.  Everything is generated on the CPU in float32 with
``torch.Generator().manual_seed(seed)`` in a fixed draw order:
q, k, v, beta-logits, gates, h0.

Workloads (name: path, sizes, distributions):
  gdn_f32_small   gdn fp32   B=1 H=2  T=256   dk=dv=64  C=64
                  q,k ~ N(0,1) then L2-normalised per (b,t,h); v ~ N(0,1);
                  beta = sigmoid(N(0,1)); a ~ U[0.9,0.999] per token-head,
                  g = ln a; zero initial state
  la_bf16         decay_la bf16  B=2 H=8 T=4096 dk=dv=128 C=64
                  q,k,v ~ N(0,1) * 128^-1/2; g[b,t,h] = ln(1 - 2^(-5-h));
                  no beta; zero initial state
  gdn_bf16        gdn bf16   B=4 H=16 T=8192 dk=dv=128 C=64
                  as gdn_f32_small; h0 ~ 0.1 * N(0,1) (fp32)
  kda_bf16        kda bf16   B=2 H=16 T=8192 dk=dv=128 C=64
                  L2-normalised q,k; v ~ N(0,1); beta = sigmoid(N(0,1));
                  a ~ U[0.9,0.999] per channel; zero initial state
  kda_bf16_long   kda bf16   B=1 H=32 T=32768 dk=dv=128 C=64, as kda_bf16;
                  stress variant: a ~ U[0.8,0.999]
  gdn_bf16_long   gdn bf16   B=1 H=32 T=32768 dk=dv=128 C=64, as gdn_bf16
                  with a zero initial state (the GDN line of the T=32k metric)

h0 is returned in the library's state layout [B, H, Dk, Dv] (fp32).

generate_raw() draws the raw projections the input prologue takes instead
(unnormalised q, k; beta logits; the scalar gate's input and its per-head
A_log, dt_bias as the Gated DeltaNet layer initialises them).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Dict, List, Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "kda" | "gdn" | "decay_la"
    dtype: str           # "f32" | "bf16"
    B: int
    H: int
    T: int
    Dk: int
    Dv: int
    C: int = 64
    gate_lo: float = 0.9
    gate_hi: float = 0.999
    h0_std: float = 0.0  # 0 -> zero initial state
    seed: int = 0

    @property
    def token_heads(self) -> int:
        return self.B * self.T * self.H

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "gdn_f32_small": Workload("gdn_f32_small", "gdn", "f32", 1, 2, 256, 64, 64),
    "la_bf16": Workload("la_bf16", "decay_la", "bf16", 2, 8, 4096, 128, 128),
    "gdn_bf16": Workload("gdn_bf16", "gdn", "bf16", 4, 16, 8192, 128, 128, h0_std=0.1),
    "kda_bf16": Workload("kda_bf16", "kda", "bf16", 2, 16, 8192, 128, 128),
    "kda_bf16_long": Workload("kda_bf16_long", "kda", "bf16", 1, 32, 32768, 128, 128),
    "kda_bf16_long_stress": Workload("kda_bf16_long_stress", "kda", "bf16", 1, 32, 32768,
                                     128, 128, gate_lo=0.8),
    "gdn_bf16_long": Workload("gdn_bf16_long", "gdn", "bf16", 1, 32, 32768, 128, 128),
    # one GPU's share of kda_bf16_long when its heads are split over 8 GPUs
    "kda_bf16_long_h4": Workload("kda_bf16_long_h4", "kda", "bf16", 1, 4, 32768, 128, 128),
}


def _l2norm(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)


def io_torch_dtype(w: Workload) -> torch.dtype:
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def generate(w: Workload, device: Optional[str] = None) -> Dict[str, Optional[torch.Tensor]]:
    """Draw the inputs of workload ``w``.  Returns CPU tensors unless a device
    is given: q, k [B,T,H,Dk] and v [B,T,H,Dv] in the I/O dtype; g fp32
    ([B,T,H,Dk] for kda, else [B,T,H]); beta fp32 [B,T,H] or None; h0 fp32
    [B,H,Dk,Dv] or None."""
    gen = torch.Generator().manual_seed(w.seed)
    B, T, H, Dk, Dv = w.B, w.T, w.H, w.Dk, w.Dv
    q = torch.randn(B, T, H, Dk, generator=gen)
    k = torch.randn(B, T, H, Dk, generator=gen)
    v = torch.randn(B, T, H, Dv, generator=gen)
    if w.kind == "decay_la":
        s = 1.0 / math.sqrt(Dk)
        q, k, v = q * s, k * s, v * s
        beta = None
        gam = 1.0 - torch.pow(2.0, -5.0 - torch.arange(H, dtype=torch.float64))
        g = torch.log(gam).to(torch.float32).view(1, 1, H).expand(B, T, H).contiguous()
    else:
        q, k = _l2norm(q), _l2norm(k)
        beta = torch.sigmoid(torch.randn(B, T, H, generator=gen))
        gshape = (B, T, H, Dk) if w.kind == "kda" else (B, T, H)
        a = torch.rand(gshape, generator=gen) * (w.gate_hi - w.gate_lo) + w.gate_lo
        g = torch.log(a)
    h0 = None
    if w.h0_std > 0:
        h0 = torch.randn(B, H, Dk, Dv, generator=gen) * w.h0_std
    dt = io_torch_dtype(w)
    out = {"q": q.to(dt).contiguous(), "k": k.to(dt).contiguous(), "v": v.to(dt).contiguous(),
           "g": g.contiguous(), "beta": beta, "h0": h0}
    if device is not None:
        out = {n: (t.to(device) if t is not None else None) for n, t in out.items()}
    return out


def generate_raw(w: Workload, device: Optional[str] = None) -> Dict[str, Optional[torch.Tensor]]:
    """Raw inputs for the input prologue, in the draw order q, k, row scales,
    v, beta logits, gates, A_log, h0:
      q, k ~ N(0,1) times a per-(b,t,h) scale U[0.25, 4] (not normalised);
      v ~ N(0,1); beta logits ~ N(0,1) (None for decay_la);
      kda: g = ln U[gate_lo, gate_hi] per channel (no gate generation);
      gdn, decay_la: gate input a ~ N(0,1), A_log = ln U[0.01, 16] and
      dt_bias = 1 per head (the layer's initialisation on the Gated DeltaNet
      page, section "输入投影").
    Returns the dict of generate() plus "A_log" and "dt_bias" (fp32 [H] or
    None)."""
    gen = torch.Generator().manual_seed(w.seed)
    B, T, H, Dk, Dv = w.B, w.T, w.H, w.Dk, w.Dv
    q = torch.randn(B, T, H, Dk, generator=gen)
    k = torch.randn(B, T, H, Dk, generator=gen)
    sc = torch.rand(2, B, T, H, 1, generator=gen) * 3.75 + 0.25
    q, k = q * sc[0], k * sc[1]
    v = torch.randn(B, T, H, Dv, generator=gen)
    beta = None if w.kind == "decay_la" else torch.randn(B, T, H, generator=gen)
    A_log = dt_bias = None
    if w.kind == "kda":
        a = torch.rand(B, T, H, Dk, generator=gen) * (w.gate_hi - w.gate_lo) + w.gate_lo
        g = torch.log(a)
    else:
        g = torch.randn(B, T, H, generator=gen)
        A_log = torch.log(torch.rand(H, generator=gen) * (16.0 - 0.01) + 0.01)
        dt_bias = torch.ones(H)
    h0 = None
    if w.h0_std > 0:
        h0 = torch.randn(B, H, Dk, Dv, generator=gen) * w.h0_std
    dt = io_torch_dtype(w)
    out = {"q": q.to(dt).contiguous(), "k": k.to(dt).contiguous(), "v": v.to(dt).contiguous(),
           "g": g.contiguous(), "beta": beta, "h0": h0, "A_log": A_log, "dt_bias": dt_bias}
    if device is not None:
        out = {n: (t.to(device) if t is not None else None) for n, t in out.items()}
    return out


def packed_lengths(T: int, seed: int = 7, lo: int = 64, hi: int = 4096) -> List[int]:
    """Sequence lengths for a packed batch of T tokens: seeded draws uniform
    in [lo, hi] until T is used up (the last sequence takes the remainder)."""
    rng = torch.Generator().manual_seed(seed)
    lengths, left = [], T
    while left > 0:
        n = min(left, int(torch.randint(lo, hi + 1, (1,), generator=rng).item()))
        lengths.append(n)
        left -= n
    return lengths
