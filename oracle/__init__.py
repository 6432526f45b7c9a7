"""CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and this
package imports nothing from the GPU library: the two share no code.

Contents
  recurrence.c   the definition: a token-by-token fp64 recurrence (C, pthreads)
  chunked.py     the chunk-form algorithm in fp64 numpy, exposing every
                 intermediate (gamma, K+, K-, A, T, W, U, state per chunk)
  prologue.py    the input prologue (q/k L2 norm, scale, beta sigmoid, scalar
                 gate generation) in fp64 numpy
  backward.py    the gradients of the token recurrence (its reverse sweep),
                 fp64 numpy

Page keys used in citations (title of the page, then the section):
  [SD]   "TileLang 实战：KDA 从零到一--标量衰减"
  [KDA]  "TileLang 实战：KDA 从零到一–Kimi Delta Attention"
  [GDN]  "Gated DeltaNet"
  [DPLR] "RNN的复兴04:线性注意力并行计算DPLR"
  [EVO]  "07 · linear 路线（二）：衰减机制的演进"

Parity status: every function here is pinned by a ``-m "not gpu"`` test
(closed forms, brute force, printed values); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "recurrence.c")
_LIB = os.path.join(_HERE, "liboracle.so")

KIND_KDA, KIND_GDN, KIND_LA = 0, 1, 2
_KINDS = {"kda": KIND_KDA, "gdn": KIND_GDN, "decay_la": KIND_LA}


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the C oracle with gcc (plain -O2; no fast-math, so fp64
    arithmetic keeps IEEE semantics)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", out, src,
           "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    return out


_lib_cache = {}


def load(path: str = _LIB) -> ctypes.CDLL:
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path) or (path == _LIB and os.path.getmtime(path) < os.path.getmtime(_SRC)):
        if path != _LIB:
            raise FileNotFoundError(path)
        build()
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.oracle_forward.argtypes = [ctypes.c_int, dp, dp, dp, dp, dp, dp, dp, dp,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.oracle_forward.restype = ctypes.c_int
    lib.oracle_default_threads.restype = ctypes.c_int
    _lib_cache[path] = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor (CPU) -> numpy, exact upcast
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def recurrence(kind, q, k, v, g, beta=None, h0=None, nthreads: int = 0,
               lib_path: str = _LIB) -> Tuple[np.ndarray, np.ndarray]:
    """Token-by-token fp64 forward of the gated delta rule.

    kind: "kda" | "gdn" | "decay_la" (or 0/1/2).
    q, k: [B,T,H,Dk]; v: [B,T,H,Dv]; g: [B,T,H,Dk] (kda) or [B,T,H];
    beta: [B,T,H] (unused for decay_la); h0: [B,H,Dv,Dk] in the pages'
    orientation (S in R^{dv x dk}), or None for a zero initial state.
    Returns (o [B,T,H,Dv], hT [B,H,Dv,Dk]) as float64, hT in the same
    orientation as h0.
    """
    kind = _KINDS.get(kind, kind)
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    beta, h0 = _f64(beta), _f64(h0)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, T, H)
    if kind == KIND_KDA:
        assert g.shape == (B, T, H, Dk)
    else:
        assert g.shape == (B, T, H)
    if kind != KIND_LA:
        assert beta is not None and beta.shape == (B, T, H)
    else:
        beta = None
    if h0 is not None:
        assert h0.shape == (B, H, Dv, Dk)
    o = np.zeros((B, T, H, Dv), dtype=np.float64)
    hT = np.zeros((B, H, Dv, Dk), dtype=np.float64)
    lib = load(lib_path)
    rc = lib.oracle_forward(kind, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                            _ptr(h0), _ptr(o), _ptr(hT), B, T, H, Dk, Dv, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_forward failed with code {rc}")
    return o, hT


def default_threads() -> int:
    return int(load().oracle_default_threads())
