"""GPU parity of 128-token chunks with 64-token sub-chunks (C = 128 through
the C ABI) against the fp64 oracle.

Page: "TileLang 实战：KDA 从零到一–Kimi Delta Attention", section 2.3 (the
sub-chunk safeguard): gamma is re-based at each sub-chunk's start, so the
largest 2^-gamma the kernels form is that of 64 positions, not 128; the
128-row UT system is solved by block elimination over the two sub-chunks.

The oracle is independent of the sub-chunking: its chunk form at C = 128
(oracle/chunked.py) forms the whole 128 x 128 A, Aqk and T in fp64, and the
token recurrence gives o and hT.  Tolerances are the forward's
(test_gpu_parity): fp32 max-rel 1e-4; bf16 rel-L2 and max-rel 2e-2 and
max/rms <= 2e-2 + 3 bf16 floors.  fp32 at Dk = 128 is not built at C = 128
and must be refused.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle import chunked
from oracle import prologue as opro
from delta_rule_rnn_amd.inputs import WORKLOADS, Workload, generate, generate_raw

from .test_gpu_parity import assert_close, bf16_floor, check_full, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
C2 = 128


def _ops():
    import delta_rule_rnn_amd as dra
    return dra


def run128(w, x, **kw):
    dra = _ops()
    d = to_dev(x)
    o, hT = dra.forward(w.kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], chunk_size=C2, **kw)
    torch.cuda.synchronize()
    return o, hT


BUILT = [("bf16", 64), ("bf16", 128), ("f32", 64)]


@pytest.mark.parametrize("T", [1, 40, 64, 65, 128, 129, 300, 1000])
@pytest.mark.parametrize("dt,D", BUILT, ids=lambda v: str(v))
@pytest.mark.parametrize("kind", ["kda", "gdn", "decay_la"])
def test_chunk128_parity(kind, dt, D, T):
    """Every element against the recurrence: full 128-token chunks, a ragged
    tail whose second sub-chunk is partly filled (65, 129, 300, 1000) or
    empty (1, 40, 64), and a nonzero initial state."""
    B = 1 if T >= 1000 else 2
    w = Workload(f"c128_{kind}_{dt}_{D}_{T}", kind, dt, B=B, H=2, T=T, Dk=D, Dv=D, h0_std=0.1,
                 seed=T + D + len(kind))
    x = generate(w)
    o, hT = run128(w, x)
    check_full(w, x, o, hT)


def _per_chunk(a, NT, C):
    """[B, T, H, X] -> [B, H, NT, C, X], rows past T zero."""
    pad = np.zeros((a.shape[0], NT * C - a.shape[1]) + a.shape[2:])
    a = np.concatenate([a, pad], 1)
    return np.moveaxis(a.reshape(a.shape[0], NT, C, a.shape[2], a.shape[3]), 3, 1)


@pytest.mark.parametrize("dt,D", BUILT, ids=lambda v: str(v))
@pytest.mark.parametrize("kind", ["kda", "gdn", "decay_la"])
def test_chunk128_records(kind, dt, D):
    """The chunk-parallel kernel alone at C = 128: every block of every
    128-row record (W, U, Q~, Kbar, the whole 128 x 128 Aqk including the
    cross-sub-chunk block and the zero block above it, phi) against the
    oracle's chunk form at C = 128, which never splits the chunk.  This pins
    the sub-chunk assembly (gamma re-basing, the block elimination of T) to
    the plain definition.  Bound: fp32 2e-5 of the rms (max), bf16 rel-L2
    2e-2."""
    dra = _ops()
    T = 300
    w = Workload(f"rec128_{kind}", kind, dt, B=1, H=2, T=T, Dk=D, Dv=D, seed=41)
    x = generate(w)
    d = to_dev(x)
    ws = dra.intra(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], C2)
    torch.cuda.synchronize()
    io = torch.float32 if dt == "f32" else torch.bfloat16
    rec = dra.unpack_records(ws, 1, T, 2, D, D, io, C2)
    ref = chunked.chunk_forward(kind, x["q"], x["k"], x["v"], x["g"], x["beta"], None, C2)
    NT = -(-T // C2)
    pc = lambda a: _per_chunk(a, NT, C2)
    checks = [("Qt", pc(ref.prep["Qp"]), rec["Qt"]),
              ("KbT", np.swapaxes(pc(ref.prep["Kbar"]), -1, -2), rec["KbT"]),
              ("Aqk", pc(ref.Aqk), rec["Aqk"]),
              ("phi", np.moveaxis(ref.prep["phi"], 2, 1), rec["phi"])]
    if kind != "decay_la":
        checks += [("W", pc(ref.W), rec["W"]), ("UT", np.swapaxes(pc(ref.U), -1, -2), rec["UT"])]
    else:
        checks += [("UT", np.swapaxes(pc(x["v"].double().numpy()), -1, -2), rec["UT"])]
    tol = 2e-5 if dt == "f32" else 2e-2
    for name, r, got in checks:
        got = got.float().cpu().numpy()
        assert np.all(np.isfinite(got)), f"{name}: non-finite"
        diff = got - r
        rms = max(np.sqrt(np.mean(r ** 2)), 1e-30)
        e = (np.max(np.abs(diff)) if dt == "f32" else np.sqrt(np.mean(diff ** 2))) / rms
        assert e <= tol, f"{name}: err {e:.3e}"
    # the first sub-chunk's rows hold exact zeros against the second's keys
    assert float(rec["Aqk"][..., :64, 64:].abs().max()) == 0.0


def test_chunk128_resume_and_determinism():
    """Splitting a sequence at a 128-token boundary and resuming from hT gives
    the same output as one call, and two calls are bit-identical."""
    dra = _ops()
    w = Workload("c128_resume", "kda", "bf16", B=1, H=2, T=512, Dk=128, Dv=128, seed=8)
    d = to_dev(generate(w))
    o, hT = dra.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk_size=C2)
    o2, hT2 = dra.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk_size=C2)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(hT, hT2)
    cut = 256
    sl = lambda t, a, b: t[:, a:b].contiguous()
    oa, ha = dra.kda_fwd(*(sl(d[n], 0, cut) for n in ("q", "k", "v", "g", "beta")), chunk_size=C2)
    ob, hb = dra.kda_fwd(*(sl(d[n], cut, w.T) for n in ("q", "k", "v", "g", "beta")), h0=ha, chunk_size=C2)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([oa, ob], 1), o)
    assert torch.equal(hb, hT)


def test_chunk128_range_flags():
    """The range flags at C = 128 describe the sub-chunks: constant gates
    a = 0.85 give -gamma = 15.0 (log2) over 64 positions, below the fp16 flag
    at 16, although a whole 128-token chunk would reach 30; a = 0.7 and a =
    0.2 raise the flags as at C = 64 (33 >= 16; 148 >= 126)."""
    dra = _ops()
    w = Workload("flags128", "kda", "bf16", B=1, H=1, T=128, Dk=64, Dv=64, seed=9)
    for a, expect in ((0.95, 0), (0.85, 0), (0.7, 1), (0.2, 3)):
        x = to_dev(generate(w))
        g = torch.full_like(x["g"], float(np.log(a)))
        flags = torch.zeros(1, dtype=torch.int32, device=DEV)
        dra.kda_fwd(x["q"], x["k"], x["v"], g, x["beta"], None, chunk_size=C2, flags=flags)
        torch.cuda.synchronize()
        assert flags.item() == expect, (a, flags.item())


def test_chunk128_stress_gate():
    """Gate-stress workload (a ~ U[0.8, 0.999]) at C = 128: the largest
    2^-gamma over whole 128-token chunks against that over 64-token
    sub-chunks (the page's table shows the same drop), the flags equal the
    C = 64 run's (the sub-chunks are the 64-token chunks), and every element
    of every chain matches the oracle."""
    dra = _ops()
    w = WORKLOADS["kda_bf16_long_stress"].with_(C=C2)
    x = generate(w)
    d = to_dev(x)
    g2 = x["g"].double().numpy() / np.log(2.0)                  # log2 gates [B, T, H, Dk]
    def max_inv(L):
        c = np.cumsum(g2.reshape(w.B, w.T // L, L, w.H, w.Dk), axis=2)
        return float(np.exp2(-c.min()))
    m128, m64 = max_inv(128), max_inv(64)
    print(f"stress: max 2^-gamma over 128-token chunks {m128:.3e}, over 64-token sub-chunks {m64:.3e}",
          flush=True)
    assert m64 < m128
    f64 = torch.zeros(1, dtype=torch.int32, device=DEV)
    f128 = torch.zeros(1, dtype=torch.int32, device=DEV)
    dra.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk_size=64, flags=f64)
    o, hT = dra.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk_size=C2, flags=f128)
    torch.cuda.synchronize()
    assert f128.item() == f64.item()
    check_full(w, x, o, hT)


@pytest.mark.parametrize("name", ["kda_bf16_long", "gdn_bf16_long", "la_bf16"])
def test_chunk128_workload_full_size(name):
    """Every element of every chain of a full-size workload at C = 128
    against one oracle pass over the whole batch; prints the margins."""
    w = WORKLOADS[name].with_(C=C2)
    x = generate(w)
    o, hT = run128(w, x)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(hT).all())
    h0 = None if x["h0"] is None else x["h0"].transpose(-1, -2)
    ro, rs = oracle.recurrence(w.kind, x["q"], x["k"], x["v"], x["g"], x["beta"], h0)
    got = o.float().cpu().numpy()
    del o
    eo = assert_close(got, ro, w.dtype, f"{name} C=128 output")
    fl = bf16_floor(ro)
    del got, ro
    es = assert_close(hT.cpu().numpy(), np.swapaxes(rs, -1, -2), w.dtype, f"{name} C=128 state")
    print(f"margins {name} (C=128): o rel-L2 {eo[1]:.2e}/2e-2, max-rel {eo[0]:.2e}/2e-2, "
          f"max/rms {eo[2]:.2e}/{2e-2 + 3 * fl:.2e} (floor {fl:.2e}); hT rel-L2 {es[1]:.2e}, max-rel {es[0]:.2e}",
          flush=True)


@pytest.mark.parametrize("kind,dt,D", [("kda", "bf16", 128), ("gdn", "f32", 64), ("decay_la", "bf16", 64)])
def test_chunk128_prologue(kind, dt, D):
    """The fused input prologue at C = 128 against the oracle's prologue and
    recurrence."""
    dra = _ops()
    w = Workload(f"{kind}_raw128", kind, dt, B=2, H=3, T=300, Dk=D, Dv=D, h0_std=0.1, seed=52)
    x = generate_raw(w)
    d = to_dev(x)
    gate = x["A_log"] is not None
    gp = dra.Prologue(qk_l2norm=True, scale=0.5, beta_sigmoid=x["beta"] is not None,
                      A_log=d["A_log"] if gate else None, dt_bias=d["dt_bias"] if gate else None)
    o, hT = dra.forward(kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], prologue=gp, chunk_size=C2)
    torch.cuda.synchronize()
    q, k, g, b = opro.apply(kind, x["q"], x["k"], x["g"], x["beta"], qk_l2norm=True, scale=0.5,
                            beta_sigmoid=x["beta"] is not None, beta_x2=False,
                            A_log=x["A_log"] if gate else None, dt_bias=x["dt_bias"] if gate else None)
    ro, rs = oracle.recurrence(kind, q, k, x["v"], g, b, x["h0"].transpose(-1, -2).contiguous())
    assert_close(o.float().cpu().numpy(), ro, dt, f"{kind} C=128 prologue output")
    assert_close(hT.cpu().numpy(), np.swapaxes(rs, -1, -2), dt, f"{kind} C=128 prologue state")


def test_chunk128_refused_where_not_built():
    """fp32 at Dk = 128 and every entry point other than the dense forward
    (packed sequences, backward) refuse C = 128 with DR_ERR_UNSUPPORTED."""
    dra = _ops()
    w = Workload("c128_f32_128", "gdn", "f32", B=1, H=1, T=130, Dk=128, Dv=128, seed=3)
    d = to_dev(generate(w))
    with pytest.raises(dra.DeltaRuleError, match="unsupported"):
        dra.gdn_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk_size=C2)
    wb = Workload("c128_bf16", "gdn", "bf16", B=1, H=1, T=130, Dk=64, Dv=64, seed=3)
    d = to_dev(generate(wb))
    cu = torch.tensor([0, 60, 130], dtype=torch.int32, device=DEV)
    with pytest.raises(dra.DeltaRuleError):
        dra.forward_varlen("gdn", d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu, chunk_size=C2)
    with pytest.raises(dra.DeltaRuleError):
        dra.backward("gdn", d["q"], d["k"], d["v"], d["g"], d["beta"], do=torch.ones_like(d["v"]), chunk_size=C2)
