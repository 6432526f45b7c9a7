"""CPU tests of the C ABI: the library loads, exports every declared symbol,
sizes its workspace as documented and rejects bad arguments on the host
before any GPU call (no compute call is made here)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "deltarule.h")


@pytest.fixture(scope="module")
def lib():
    from delta_rule_rnn_amd import _lib
    if not os.environ.get("DR_LIBRARY") and not os.path.exists(_lib.LIB_PATH):
        from delta_rule_rnn_amd.build import build_library
        build_library()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_header_and_binding_agree():
    from delta_rule_rnn_amd import _lib
    decl = declared_functions()
    assert decl == sorted(_lib.SIGNATURES), (decl, sorted(_lib.SIGNATURES))


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.dr_abi_version() == 7


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5):
        assert lib.dr_status_string(s)
    assert lib.dr_status_string(7) == b"unknown status"


def test_workspace_sizes(lib, monkeypatch):
    # one record per (b, h, chunk); bf16 D=128 record: (3*64*128 + 64*64 + 128*64)*2 + 128*4
    rec = lib.dr_record_bytes(128, 128, 64, 1)
    assert rec == ((3 * 64 * 128 + 64 * 64 + 128 * 64) * 2 + 128 * 4 + 255) // 256 * 256
    assert lib.dr_record_workspace_bytes(0, 2, 130, 3, 128, 128, 64, 1) == 2 * 3 * 3 * rec
    assert lib.dr_workspace_bytes(1, 1, 0, 1, 64, 64, 64, 0) == 0
    # segment-parallel forward: q_eff of every chunk, then [M | N] (fp32) and
    # the entry state (I/O dtype) of every segment; 6 chains of 3 chunks give
    # one-chunk segments (about 256 workgroups wanted)
    up = lambda x: (x + 255) // 256 * 256
    chains, NT, NS, D = 6, 3, 3, 128
    want = up(chains * NT * 64 * D * 2) + up(chains * NS * D * 2 * D * 4) + up(chains * NS * D * D * 2)
    assert lib.dr_segment_workspace_bytes(0, 2, 130, 3, 128, 128, 64, 1) == want
    # not built for fp32 at D = 128
    assert lib.dr_segment_workspace_bytes(0, 2, 130, 3, 128, 128, 64, 0) == 0
    # the forward's own workspace: the segment-parallel path's by default,
    # the record path's with DR_FWD_PATH=records and where the segment path
    # is not built
    assert lib.dr_workspace_bytes(0, 2, 130, 3, 128, 128, 64, 1) == want
    assert lib.dr_workspace_bytes(0, 2, 130, 3, 128, 128, 64, 0) == 2 * 3 * 3 * lib.dr_record_bytes(128, 128, 64, 0)
    monkeypatch.setenv("DR_FWD_PATH", "records")
    assert lib.dr_workspace_bytes(0, 2, 130, 3, 128, 128, 64, 1) == 2 * 3 * 3 * rec
    assert lib.dr_record_bytes(96, 96, 64, 1) == 0
    assert lib.dr_record_bytes(128, 64, 64, 1) == 0
    assert lib.dr_record_bytes(128, 128, 32, 1) == 0


def test_workspace_sizes_chunk128(lib):
    """128-token chunks: one 128-row record per (b, h, chunk) with the same
    blocks (W, Q~, Kbar^T, the 128 x 128 Aqk, U^T, phi); the dense forward
    only, not built for fp32 at D = 128."""
    rec = lib.dr_record_bytes(128, 128, 128, 1)
    assert rec == ((3 * 128 * 128 + 128 * 128 + 128 * 128) * 2 + 128 * 4 + 255) // 256 * 256
    assert lib.dr_record_bytes(64, 64, 128, 0) == ((3 * 128 * 64 + 128 * 128 + 64 * 128) * 4 + 64 * 4 + 255) // 256 * 256
    assert lib.dr_record_bytes(128, 128, 128, 0) == 0
    # T = 300 is 3 chunks of 128; the forward takes the record path
    assert lib.dr_record_workspace_bytes(0, 2, 300, 3, 128, 128, 128, 1) == 2 * 3 * 3 * rec
    assert lib.dr_workspace_bytes(0, 2, 300, 3, 128, 128, 128, 1) == 2 * 3 * 3 * rec
    assert lib.dr_segment_workspace_bytes(0, 2, 300, 3, 128, 128, 128, 1) == 0
    # packed sequences and the backward take C = 64 only
    assert lib.dr_workspace_bytes_varlen(0, 2, 300, 1, 64, 64, 128, 1) == 0
    assert lib.dr_backward_workspace_bytes(1, 1, 128, 2, 64, 64, 128, 1) == 0
    assert lib.dr_backward_varlen_workspace_bytes(1, 2, 128, 2, 64, 64, 128, 1, 0) == 0


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first


@pytest.mark.parametrize("case,expect", [
    (dict(B=0), -1), (dict(H=0), -1), (dict(T=-1), -1), (dict(dtype=5), -1),
    (dict(Dk=96, Dv=96), -2), (dict(Dk=128, Dv=64), -2), (dict(C=32), -2), (dict(C=96), -2),
    (dict(C=128, Dk=128, Dv=128, dtype=0), -2), (dict(C=128, q=None), -1), (dict(C=128, ws_bytes=100), -4),
    (dict(q=None), -1), (dict(beta=None), -1), (dict(q=FAKE + 4), -1), (dict(o=FAKE + 8), -1),
    (dict(ws=None), -4), (dict(ws_bytes=100), -4),
])
def test_kda_fwd_rejects(lib, case, expect):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, o=FAKE, hT=None, B=1, T=64, H=1,
             Dk=64, Dv=64, C=64, dtype=1, ws=FAKE, ws_bytes=1 << 30, flags=None, stream=None)
    a.update(case)
    st = lib.kda_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["o"], a["hT"], a["B"],
                     a["T"], a["H"], a["Dk"], a["Dv"], a["C"], a["dtype"], a["ws"], a["ws_bytes"],
                     a["flags"], a["stream"])
    assert st == expect


def test_noalloc_limit_is_checked_on_the_host(lib):
    """dr_forward_noalloc: bad sizes and problems larger than the static
    scratch array are rejected before any device call."""
    cap = lib.dr_noalloc_scratch_bytes()
    assert cap == 64 << 20
    args = lambda B, T, H: (0, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, B, T, H, 128, 128, 64, 1,
                            None, None, None)
    assert lib.dr_forward_noalloc(*args(0, 64, 1)) == -1
    assert lib.dr_forward_noalloc(5, *args(1, 64, 1)[1:]) == -1
    T = 64
    while lib.dr_workspace_bytes(0, 1, T, 1, 128, 128, 64, 1) <= cap:
        T *= 2
    st = lib.dr_forward_noalloc(*args(1, T, 1))
    assert st == -5 and b"static scratch" in lib.dr_status_string(st)


def test_other_entry_points_reject(lib):
    assert lib.decay_la_fwd(FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 1, 64, 1, 64, 64, 64, 1, None, 0,
                            None) == -4
    assert lib.gdn_fwd(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, 1, 64, 1, 64, 64, 64, 1, FAKE,
                       1 << 30, None, None) == -1
    assert lib.dr_chunk_cumsum(FAKE, FAKE, 1, 64, 1, 0, 64, None) == -1
    assert lib.dr_chunk_cumsum(FAKE, FAKE, 1, 64, 1, 4, 32, None) == -2
    assert lib.dr_chunk_cumsum(FAKE, FAKE, 1, 64, 1, 4, 64, None) == -1   # aliasing
    assert lib.dr_kda_prep(FAKE, FAKE, FAKE, None, None, None, None, None, 1, 64, 1, 96, 64, 1, None,
                           None) == -2
    assert lib.dr_intra(3, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 1, 64, 64, 64, 1, FAKE, 1 << 30, None,
                        None) == -1
    assert lib.dr_inter(0, None, FAKE, None, 1, 64, 1, 64, 64, 64, 1, FAKE, 10, None) == -4
    # decode: state required, sizes as for the forward, aligned pointers
    assert lib.kda_decode(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 1, 1, 128, 128, 1, None) == -1
    assert lib.gdn_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 96, 96, 1, None) == -2
    assert lib.gdn_decode(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1, 1, 1, 64, 64, 1, None) == -1
    assert lib.decay_la_decode(FAKE, FAKE, FAKE, FAKE, FAKE + 4, FAKE, 1, 1, 1, 64, 64, 1, None) == -1
    assert lib.decay_la_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 64, 64, 2, None) == -1
    # packed sequences: cu_seqlens and N >= 1 required, workspace sized by its own query
    assert lib.kda_fwd_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, None, 2, None, FAKE, None, 128, 1, 64, 64, 64, 1,
                              FAKE, 1 << 30, None, None) == -1
    assert lib.gdn_fwd_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None, FAKE, None, 128, 1, 64, 64, 64, 1,
                              FAKE, 1 << 30, None, None) == -1
    assert lib.decay_la_fwd_varlen(FAKE, FAKE, FAKE, FAKE, FAKE + 2, 2, None, FAKE, None, 128, 1, 64, 64, 64,
                                   1, FAKE, 1 << 30, None, None) == -1
    need = lib.dr_workspace_bytes_varlen(0, 2, 128, 1, 64, 64, 64, 1)
    assert need > 0 and lib.dr_workspace_bytes_varlen(0, 0, 128, 1, 64, 64, 64, 1) == 0
    assert lib.kda_fwd_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, None, FAKE, None, 128, 1, 64, 64, 64, 1,
                              FAKE, need - 1, None, None) == -4
    # decode with no tokens touches nothing
    assert lib.kda_decode(None, None, None, None, None, None, None, 1, 0, 1, 64, 64, 1, None) == 0
    # nothing to do: T = 0 and no final state requested
    assert lib.kda_fwd(None, None, None, None, None, None, None, None, 1, 0, 1, 64, 64, 64, 1, None, 0,
                       None, None) == 0


def test_python_binding_requires_library(tmp_path, monkeypatch):
    """The product path fails loudly (no CPU fallback) when the library is missing."""
    from delta_rule_rnn_amd import _lib
    monkeypatch.setattr(_lib, "_LIB", None)
    with pytest.raises(_lib.LibraryMissing):
        _lib.load(str(tmp_path / "nope.so"))


def test_prologue_rejects(lib):
    """Bad prologues are refused on the host, before any launch."""
    from delta_rule_rnn_amd._lib import DrPrologue
    base = dict(B=1, T=64, H=1, D=64)

    def fwd(kind, pro):
        return lib.dr_forward(kind, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, base["B"], base["T"],
                              base["H"], base["D"], base["D"], 64, 1, ctypes.addressof(pro), FAKE, 1 << 30, None,
                              None)

    nan = float("nan")
    assert fwd(1, DrPrologue(0x10, 1.0, None, None)) == -1                 # unknown bit
    assert fwd(1, DrPrologue(0x4, 1.0, None, None)) == -1                  # x2 without sigmoid
    assert fwd(1, DrPrologue(0x0, nan, None, None)) == -1                  # non-finite scale
    assert fwd(1, DrPrologue(0x8, 1.0, None, None)) == -1                  # gate without A_log
    assert fwd(1, DrPrologue(0x8, 1.0, FAKE + 2, None)) == -1              # misaligned A_log
    assert fwd(0, DrPrologue(0x8, 1.0, FAKE, None)) == -2                  # per-channel gate: not defined
    assert fwd(2, DrPrologue(0x2, 1.0, None, None)) == -1                  # decay_la has no beta
    assert fwd(3, DrPrologue(0x0, 1.0, None, None)) == -1                  # bad kind
    pro = DrPrologue(0x10, 1.0, None, None)
    assert lib.dr_decode(0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 64, 64, 1,
                         ctypes.addressof(pro), None) == -1
    assert lib.dr_forward_varlen(1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None, FAKE, None, 64, 1, 64, 64, 64, 1,
                                 ctypes.addressof(pro), FAKE, 1 << 30, None, None) == -1
    # the binding refuses a dt_bias without A_log before calling the library
    import torch
    from delta_rule_rnn_amd import DeltaRuleError, Prologue
    with pytest.raises(DeltaRuleError):
        Prologue(dt_bias=torch.zeros(1)).to_c(1)


def test_backward_rejects(lib):
    """dr_backward refuses bad arguments on the host, before any launch."""
    need = lib.dr_backward_workspace_bytes(1, 1, 128, 2, 64, 64, 64, 1)
    assert need > 0 and lib.dr_backward_workspace_bytes(1, 1, 128, 2, 96, 96, 64, 1) == 0

    def bwd(kind=1, dout=FAKE, dq=FAKE, dbeta=FAKE, ws=FAKE, wsb=1 << 40, D=64, T=128, dg=FAKE, q=FAKE):
        return lib.dr_backward(kind, q, FAKE, FAKE, FAKE, FAKE, None, dout, None, dq, FAKE, FAKE, dg, dbeta, None,
                               1, T, 2, D, D, 64, 1, ws, wsb, None)

    assert bwd(kind=3) == -1
    assert bwd(dout=None) == -1
    assert bwd(dq=None) == -1
    assert bwd(dg=None) == -1
    assert bwd(dbeta=None) == -1                 # gdn needs dbeta
    assert bwd(q=FAKE + 8) == -1                 # misaligned
    assert bwd(D=96) == -2
    assert bwd(ws=None) == -4
    assert bwd(wsb=need - 1) == -4


def test_backward_varlen_rejects(lib):
    """dr_backward_varlen refuses bad arguments on the host, before any launch."""
    need = lib.dr_backward_varlen_workspace_bytes(1, 3, 200, 2, 64, 64, 64, 1, 0)
    with_pro = lib.dr_backward_varlen_workspace_bytes(1, 3, 200, 2, 64, 64, 64, 1, 1)
    assert 0 < need < with_pro
    # more sequences: more chunk slots (ceil(T/C) + N per head)
    assert lib.dr_backward_varlen_workspace_bytes(1, 9, 200, 2, 64, 64, 64, 1, 0) > need
    assert lib.dr_backward_varlen_workspace_bytes(1, 0, 200, 2, 64, 64, 64, 1, 0) == 0
    assert lib.dr_backward_varlen_workspace_bytes(1, 3, 200, 2, 96, 96, 64, 1, 0) == 0

    def bwd(kind=1, cu=FAKE, N=3, dout=FAKE, dq=FAKE, dbeta=FAKE, ws=FAKE, wsb=1 << 40, D=64, T=200):
        return lib.dr_backward_varlen(kind, FAKE, FAKE, FAKE, FAKE, FAKE, cu, N, None, dout, None, dq, FAKE, FAKE,
                                      FAKE, dbeta, None, None, None, T, 2, D, D, 64, 1, None, ws, wsb, None, None)

    assert bwd(kind=3) == -1
    assert bwd(cu=None) == -1
    assert bwd(cu=FAKE + 2) == -1                # cu_seqlens must be 4-byte aligned
    assert bwd(N=0) == -1
    assert bwd(dout=None) == -1
    assert bwd(dq=None) == -1
    assert bwd(dbeta=None) == -1
    assert bwd(D=96) == -2
    assert bwd(N=1 << 30) == -2                  # grids past 2^31 workgroups, refused before any launch
    assert bwd(ws=None) == -4
    assert bwd(wsb=need - 1) == -4


def test_size_queries_at_extreme_sizes(lib, monkeypatch):
    """Every size query at INT_MAX and other extreme sizes: 0 where q would
    hold more than 2^40 elements, else the exact size (no overflow; with the
    host sanitizer build these also run under UndefinedBehaviorSanitizer)."""
    big = 2147483647
    monkeypatch.setenv("DR_FWD_PATH", "records")     # dr_workspace_bytes = the record workspace
    for B, T, H in ((1, big, 1), (big, big, big), (big, 1, 1), (1, 1, big), (2, 1 << 30, 8), (big, big, 1)):
        ok = B * T * H * 128 <= (1 << 40)
        for C in (64, 128):
            rec = lib.dr_record_bytes(128, 128, C, 1)
            want = B * H * (-(-T // C)) * rec if ok else 0
            assert lib.dr_record_workspace_bytes(1, B, T, H, 128, 128, C, 1) == want
            assert lib.dr_workspace_bytes(0, B, T, H, 128, 128, C, 1) == want
            assert (lib.dr_segment_workspace_bytes(0, B, T, H, 128, 128, C, 1) > 0) == (ok and C == 64)
        okb = B * T * H * 64 <= (1 << 40)
        assert (lib.dr_backward_workspace_bytes(1, B, T, H, 64, 64, 64, 1) > 0) == okb
        assert (lib.dr_backward_prologue_workspace_bytes(1, B, T, H, 64, 64, 64, 1) > 0) == okb
        okv = T * H * 64 <= (1 << 40) and ((-(-T // 64)) + B) * H <= big
        assert (lib.dr_workspace_bytes_varlen(0, B, T, H, 64, 64, 64, 1) > 0) == okv
        assert (lib.dr_backward_varlen_workspace_bytes(0, B, T, H, 64, 64, 64, 1, 1) > 0) == okv
    # the largest accepted problem (2^40 elements of q) and one token more
    T = (1 << 40) // (128 * 128)
    assert lib.dr_workspace_bytes(0, 1, T, 128, 128, 128, 64, 1) > 0
    assert lib.dr_workspace_bytes(0, 1, T + 1, 128, 128, 128, 64, 1) == 0
    # entry points reject the same sizes on the host
    assert lib.kda_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, big, big, big, 64, 64, 64, 1, FAKE,
                       1 << 30, None, None) == -1
