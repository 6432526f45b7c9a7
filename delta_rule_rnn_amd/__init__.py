"""Chunkwise gated-delta-rule forward (KDA / Gated DeltaNet / scalar-decay
linear attention) for AMD Instinct MI355X (gfx950).

The computation lives in libdeltarule.so (HIP kernels behind the C ABI of
include/deltarule.h); this package only marshals torch tensors into it.
Importing the package does not load the library; the first op call does, and
raises if the library has not been built.
"""
from .ops import (DeltaRuleError, Prologue, backward, backward_varlen, backward_varlen_workspace_bytes,
                  backward_workspace_bytes, chunk_cumsum, decay_la_decode, decay_la_fwd, decode, forward,
                  forward_noalloc, forward_varlen, gdn_decode, gdn_fwd, inter, intra, kda_decode, kda_fwd, kda_prep,
                  unpack_records, workspace_bytes, workspace_bytes_varlen)
from .autograd import chunk_delta_rule

__all__ = ["kda_fwd", "gdn_fwd", "decay_la_fwd", "forward", "kda_decode", "gdn_decode",
           "decay_la_decode", "decode", "forward_noalloc", "forward_varlen", "workspace_bytes_varlen", "chunk_cumsum", "kda_prep", "intra", "inter",
           "unpack_records", "workspace_bytes", "DeltaRuleError", "Prologue", "backward",
           "backward_workspace_bytes", "backward_varlen", "backward_varlen_workspace_bytes", "chunk_delta_rule"]
