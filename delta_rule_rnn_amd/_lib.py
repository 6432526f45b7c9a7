"""ctypes loader of libdeltarule.so (the C ABI of include/deltarule.h).

The library is never built on import: build it with ``__graft_entry__.build()``
(or ``python -m delta_rule_rnn_amd.build``).  A missing library raises."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdeltarule.so")

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/deltarule.h
SIGNATURES = {
    "dr_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "dr_record_bytes": (_sz, [_i, _i, _i, _i]),
    "dr_record_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "dr_segment_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "dr_forward_stage": (_i, [_i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp,
                              _sz, _vp, _vp]),
    "kda_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp, _vp]),
    "gdn_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp, _vp]),
    "decay_la_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "dr_workspace_bytes_varlen": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "kda_fwd_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp, _vp]),
    "gdn_fwd_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp, _vp]),
    "decay_la_fwd_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp, _vp]),
    "kda_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "gdn_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "decay_la_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "dr_forward": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _sz, _vp,
                        _vp]),
    "dr_noalloc_scratch_bytes": (_sz, []),
    "dr_forward_noalloc": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp,
                                _vp]),
    "dr_forward_varlen": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp,
                               _vp, _sz, _vp, _vp]),
    "dr_decode": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp]),
    "dr_backward_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "dr_backward": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                         _i, _i, _vp, _sz, _vp]),
    "dr_backward_prologue_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "dr_backward_prologue": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "dr_backward_varlen_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i, _i]),
    "dr_backward_varlen": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _sz, _vp, _vp]),
    "dr_chunk_cumsum": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "dr_kda_prep": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp]),
    "dr_intra": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp, _vp]),
    "dr_inter": (_i, [_i, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "dr_status_string": (ctypes.c_char_p, [_i]),
    "dr_abi_version": (_i, []),
}



class DrPrologue(ctypes.Structure):
    """struct dr_prologue of include/deltarule.h."""
    _fields_ = [("ops", ctypes.c_uint), ("scale", ctypes.c_float), ("A_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p)]


PRO_QK_L2NORM, PRO_BETA_SIGMOID, PRO_BETA_X2, PRO_GATE = 0x1, 0x2, 0x4, 0x8

_LIB = None


class LibraryMissing(RuntimeError):
    pass


def load(path: str = "") -> ctypes.CDLL:
    """Load the library once: `path`, else the file the environment variable
    DR_LIBRARY names (another build of the same sources, e.g. one with host
    sanitizers), else the in-tree build."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = path or os.environ.get("DR_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise LibraryMissing(
            f"{path} is not built; run __graft_entry__.build() (hipcc, gfx950) first")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib
