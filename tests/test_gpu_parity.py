"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (per output, o and the final state hT separately):
  fp32 I/O:  max|gpu - ref| / max|ref|  <= 1e-4
  bf16 I/O:  ||gpu - ref|| / ||ref||    <= 2e-2   (error RMS relative to the
             output RMS: the pages' kernel acceptance metric, "TileLang 实战：
             KDA 从零到一--标量衰减" section 7 item 4)
             max|gpu - ref| / max|ref| <= 2e-2   (max relative error)
  max|gpu - ref| / rms(ref) is printed too, next to its floor: the same
  quantity for the fp64 reference merely rounded to bf16, which already
  exceeds 2e-2 on the delta-rule workloads (heavy-tailed outputs), so no
  bf16-output implementation can meet that stricter reading.
Small cases compare every element; the full-size workloads run in the same
launch configuration as the benchmark and compare sampled (b, h) chains,
which the oracle computes one by one.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle import chunked
from delta_rule_rnn_amd.inputs import WORKLOADS, Workload, generate

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _ops():
    import delta_rule_rnn_amd as dra
    return dra


def to_dev(x):
    return {n: (t.to(DEV) if t is not None else None) for n, t in x.items()}


def errs(gpu: np.ndarray, ref: np.ndarray):
    """(max|d|/max|ref|, ||d||/||ref||, max|d|/rms(ref))"""
    d = np.abs(gpu - ref)
    rms = max(np.sqrt(np.mean(ref ** 2)), 1e-30)
    return (np.max(d) / max(np.max(np.abs(ref)), 1e-30), np.sqrt(np.mean(d ** 2)) / rms,
            np.max(d) / rms)


def bf16_floor(ref: np.ndarray) -> float:
    """max|bf16(ref) - ref| / rms(ref): what storing the exact result in bf16 costs."""
    r = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).double().numpy()
    return float(np.max(np.abs(r - ref)) / max(np.sqrt(np.mean(ref ** 2)), 1e-30))


def assert_close(gpu, ref, dtype: str, what: str, tol_l2=2e-2, tol_max=2e-2):
    e_max, e_l2, e_rms = errs(gpu, ref)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    if dtype == "f32":
        assert e_max <= 1e-4, f"{what}: max rel err {e_max:.3e} > 1e-4"
    else:
        assert e_l2 <= tol_l2, f"{what}: rel-L2 {e_l2:.3e} > {tol_l2}"
        assert e_max <= tol_max, f"{what}: max rel err {e_max:.3e} > {tol_max}"
    return e_max, e_l2, e_rms


def run_gpu(w: Workload, x: dict, **kw):
    dra = _ops()
    d = to_dev(x)
    o, hT = dra.forward(w.kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], **kw)
    torch.cuda.synchronize()
    return o, hT


def oracle_chains(w: Workload, x: dict, chains):
    """Oracle outputs for the selected (b, h) chains: lists of (o [T,Dv], hT [Dk,Dv])."""
    out = []
    for (b, h) in chains:
        sl = lambda t: None if t is None else t[b:b + 1, :, h:h + 1].contiguous()
        h0 = None if x["h0"] is None else x["h0"][b:b + 1, h:h + 1].transpose(-1, -2).contiguous()
        ro, rs = oracle.recurrence(w.kind, sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]),
                                   sl(x["beta"]), h0, nthreads=len(chains))
        out.append((ro[0, :, 0], rs[0, 0].T))
    return out


def check_full(w: Workload, x: dict, o, hT):
    h0 = None if x["h0"] is None else x["h0"].transpose(-1, -2)
    ro, rs = oracle.recurrence(w.kind, x["q"], x["k"], x["v"], x["g"], x["beta"], h0)
    eo = assert_close(o.float().cpu().numpy(), ro, w.dtype, f"{w.name} output")
    es = assert_close(hT.cpu().numpy(), np.swapaxes(rs, -1, -2), w.dtype, f"{w.name} state")
    fl = bf16_floor(ro) if w.dtype == "bf16" else 0.0
    print(f"{w.name}: o max-rel {eo[0]:.2e} rel-L2 {eo[1]:.2e} max/rms {eo[2]:.2e} (bf16 floor {fl:.2e});"
          f" hT max-rel {es[0]:.2e} rel-L2 {es[1]:.2e} max/rms {es[2]:.2e}", flush=True)


# ---------------------------------------------------------------------------
# small cases: every kind, dtype and head size; several chunks + ragged tail
# ---------------------------------------------------------------------------
SMALL = []
for kind in ("kda", "gdn", "decay_la"):
    for dt in ("f32", "bf16"):
        for D in (64, 128):
            SMALL.append(Workload(f"{kind}_{dt}_{D}", kind, dt, B=2, H=3, T=209, Dk=D, Dv=D,
                                  h0_std=0.1, seed=D + len(SMALL)))


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_parity(w):
    x = generate(w)
    o, hT = run_gpu(w, x)
    check_full(w, x, o, hT)


@pytest.mark.parametrize("T", [1, 17, 63, 64, 65, 128, 130])
@pytest.mark.parametrize("kind", ["kda", "gdn", "decay_la"])
def test_lengths(kind, T):
    w = Workload(f"{kind}_T{T}", kind, "bf16", B=1, H=2, T=T, Dk=128, Dv=128, h0_std=0.1, seed=T)
    x = generate(w)
    o, hT = run_gpu(w, x)
    check_full(w, x, o, hT)


def test_empty_sequence_copies_state():
    dra = _ops()
    w = Workload("kda_T0", "kda", "bf16", B=2, H=2, T=0, Dk=64, Dv=64, h0_std=1.0)
    x = to_dev(generate(w))
    o, hT = dra.kda_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 2, 64)
    assert torch.equal(hT, x["h0"])
    _, hT0 = dra.kda_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(hT0).item() == 0


def test_resume_is_exact():
    """Splitting at a chunk boundary and handing the state over through
    h0/hT gives bit-identical results (same chunks, same arithmetic)."""
    dra = _ops()
    w = Workload("kda_resume", "kda", "bf16", B=1, H=4, T=320, Dk=128, Dv=128, h0_std=0.1, seed=5)
    x = to_dev(generate(w))
    o, hT = dra.kda_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    s = 192
    cut = lambda t, a, b: t[:, a:b].contiguous()
    o1, h1 = dra.kda_fwd(cut(x["q"], 0, s), cut(x["k"], 0, s), cut(x["v"], 0, s), cut(x["g"], 0, s),
                         cut(x["beta"], 0, s), x["h0"])
    o2, h2 = dra.kda_fwd(cut(x["q"], s, 320), cut(x["k"], s, 320), cut(x["v"], s, 320),
                         cut(x["g"], s, 320), cut(x["beta"], s, 320), h1)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2], 1), o)
    assert torch.equal(h2, hT)



@pytest.mark.parametrize("kind", ["kda", "gdn", "decay_la"])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_state_pass_layouts_agree(kind, dt, monkeypatch):
    """The state pass may give each workgroup 16, 32 or 64 value columns and
    may run an L2 prefetch wave; the arithmetic of every column is the same
    in all of them, so results are bit-identical (small problems pick 16
    columns on their own, so the others are forced here)."""
    dra = _ops()
    w = Workload(f"{kind}_layouts", kind, dt, B=2, H=3, T=64 * 5 + 9, Dk=128, Dv=128, h0_std=0.1, seed=9)
    x = to_dev(generate(w))
    monkeypatch.setenv("DR_INTER_NTN", "1")
    monkeypatch.setenv("DR_INTER_PFD", "0")
    o1, h1 = dra.forward(kind, x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    torch.cuda.synchronize()
    for ntn in ("1", "2", "4"):
        for pfd in ("0", "2"):
            monkeypatch.setenv("DR_INTER_NTN", ntn)
            monkeypatch.setenv("DR_INTER_PFD", pfd)
            o2, h2 = dra.forward(kind, x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
            torch.cuda.synchronize()
            assert torch.equal(o2, o1) and torch.equal(h2, h1), f"columns {16 * int(ntn)}, prefetch {pfd}"

def test_deterministic():
    w = Workload("gdn_det", "gdn", "bf16", B=2, H=4, T=500, Dk=128, Dv=128, h0_std=0.1, seed=6)
    x = generate(w)
    o1, h1 = run_gpu(w, x)
    o2, h2 = run_gpu(w, x)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


# ---------------------------------------------------------------------------
# individual steps against the chunk-form oracle
# ---------------------------------------------------------------------------
def test_step_a1_cumsum():
    dra = _ops()
    for shape in ((2, 200, 3, 128), (2, 200, 3, 64), (2, 200, 3)):
        g = torch.log(torch.rand(shape, generator=torch.Generator().manual_seed(1)) * 0.099 + 0.9)
        got = dra.chunk_cumsum(g.to(DEV)).cpu().numpy()
        ref = chunked.chunk_log2_cumsum(g, 64)
        assert np.max(np.abs(got - ref)) <= 1e-5 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_step_a2_prep(dt):
    dra = _ops()
    w = Workload("prep", "kda", dt, B=2, H=3, T=200, Dk=128, Dv=128, seed=3)
    x = generate(w)
    d = to_dev(x)
    gam = dra.chunk_cumsum(d["g"])
    qp, kp, km, kbar, phi = dra.kda_prep(d["q"], d["k"], gam)
    torch.cuda.synchronize()
    ref = chunked.separable_prep(x["q"], x["k"], chunked.chunk_log2_cumsum(x["g"], 64), 64)
    tol = 1e-5 if dt == "f32" else 8e-3   # one rounding to the I/O dtype
    for name, got in (("Qp", qp), ("Kp", kp), ("Km", km), ("Kbar", kbar)):
        r = ref[name]
        e = np.max(np.abs(got.float().cpu().numpy() - r) / np.maximum(np.abs(r), 1e-3))
        assert e <= tol, f"{name}: {e:.3e}"
    assert np.max(np.abs(phi.cpu().numpy() - ref["phi"]) / ref["phi"]) <= 1e-5


def _record_refs(w, x):
    # the records do not depend on the initial state
    return chunked.chunk_forward(w.kind, x["q"], x["k"], x["v"], x["g"], x["beta"], None, 64)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["kda", "gdn", "decay_la"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_step_a3_records(kind, dt, D):
    """K1 alone: W, U, Q~, Kbar, Aqk and phi of every chunk against the
    chunk-form oracle's intermediates (step a3 = the UT transform).  Bound:
    fp32 1e-5 of the rms; bf16 rel-L2 2e-2 (a few bf16 roundings)."""
    dra = _ops()
    w = Workload(f"rec_{kind}", kind, dt, B=1, H=2, T=150, Dk=D, Dv=D, seed=4)
    x = generate(w)
    d = to_dev(x)
    ws = dra.intra(kind, d["q"], d["k"], d["v"], d["g"], d["beta"])
    torch.cuda.synchronize()
    io = torch.float32 if dt == "f32" else torch.bfloat16
    rec = dra.unpack_records(ws, 1, 150, 2, D, D, io)
    ref = _record_refs(w, x)
    tol = 2e-5 if dt == "f32" else 2e-2
    NT = 3
    pad = lambda a: np.concatenate([a, np.zeros((a.shape[0], NT * 64 - a.shape[1]) + a.shape[2:])], 1)
    def per_chunk(a):   # [B,T,H,X] -> [B,H,NT,64,X]
        a = pad(a)
        return np.moveaxis(a.reshape(a.shape[0], NT, 64, a.shape[2], a.shape[3]), 3, 1)
    checks = [("Qt", per_chunk(ref.prep["Qp"]), rec["Qt"]),
              ("KbT", np.swapaxes(per_chunk(ref.prep["Kbar"]), -1, -2), rec["KbT"]),
              ("Aqk", per_chunk(ref.Aqk), rec["Aqk"]),
              ("phi", np.moveaxis(ref.prep["phi"], 2, 1), rec["phi"])]
    if kind != "decay_la":
        checks += [("W", per_chunk(ref.W), rec["W"]), ("UT", np.swapaxes(per_chunk(ref.U), -1, -2), rec["UT"])]
    else:
        checks += [("UT", np.swapaxes(per_chunk(x["v"].double().numpy()), -1, -2), rec["UT"])]
    for name, r, got in checks:
        got = got.float().cpu().numpy()
        assert np.all(np.isfinite(got)), f"{name}: non-finite"
        d = got - r
        rms = max(np.sqrt(np.mean(r ** 2)), 1e-30)
        e = (np.max(np.abs(d)) if dt == "f32" else np.sqrt(np.mean(d ** 2))) / rms
        assert e <= tol, f"{name}: err {e:.3e}"


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_inter_from_records_matches_forward(dt):
    dra = _ops()
    w = Workload("split", "kda", dt, B=2, H=2, T=300, Dk=128, Dv=128, h0_std=0.1, seed=8)
    d = to_dev(generate(w))
    o, hT = dra.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    ws = dra.intra("kda", d["q"], d["k"], d["v"], d["g"], d["beta"])
    hT2 = torch.empty_like(hT)
    o2, _ = dra.inter("kda", ws, 2, 300, 2, 128, 128, d["q"].dtype, h0=d["h0"], hT=hT2)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(hT, hT2)


def test_gate_range_flags():
    """The KDA path reports chunk-local -gamma_log2 >= 16 (fp16 range of
    k 2^-gamma) and >= 126 (overflow) through the flags word."""
    dra = _ops()
    w = Workload("flags", "kda", "bf16", B=1, H=1, T=64, Dk=64, Dv=64, seed=9)
    for a, expect in ((0.95, 0), (0.7, 1), (0.2, 3)):
        x = to_dev(generate(w))
        g = torch.full_like(x["g"], float(np.log(a)))
        flags = torch.zeros(1, dtype=torch.int32, device=DEV)
        dra.kda_fwd(x["q"], x["k"], x["v"], g, x["beta"], None, flags=flags)
        torch.cuda.synchronize()
        assert flags.item() == expect, (a, flags.item())


# ---------------------------------------------------------------------------
# the five workloads at full size (sampled chains), benchmark launch config
# ---------------------------------------------------------------------------
def test_workload_gdn_f32_small_full():
    w = WORKLOADS["gdn_f32_small"]
    x = generate(w)
    o, hT = run_gpu(w, x)
    check_full(w, x, o, hT)


@pytest.mark.parametrize("name", ["la_bf16", "gdn_bf16", "kda_bf16", "kda_bf16_long",
                                  "kda_bf16_long_stress", "gdn_bf16_long"])
def test_workload_full_size_sampled(name):
    w = WORKLOADS[name]
    x = generate(w)
    print(f"{name}: inputs generated", flush=True)
    o, hT = run_gpu(w, x)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(hT).all())
    chains = [(0, 0), (w.B - 1, w.H - 1)]
    refs = oracle_chains(w, x, chains)
    for (b, h), (ro, rs) in zip(chains, refs):
        eo = assert_close(o[b, :, h].float().cpu().numpy(), ro, w.dtype, f"{name} o b={b} h={h}")
        es = assert_close(hT[b, h].cpu().numpy(), rs, w.dtype, f"{name} hT b={b} h={h}")
        print(f"{name} chain ({b},{h}): o max-rel {eo[0]:.2e} rel-L2 {eo[1]:.2e} max/rms {eo[2]:.2e}"
              f" (bf16 floor {bf16_floor(ro):.2e}); hT max-rel {es[0]:.2e} rel-L2 {es[1]:.2e}", flush=True)


def test_stress_gate_km_range():
    """Gate-stress variant (a ~ U[0.8, 0.999]): K- = k 2^-gamma stays finite
    and below the fp16 maximum 65504 (checked on the step-a2 output), and the
    flags agree."""
    dra = _ops()
    w = WORKLOADS["kda_bf16_long_stress"]
    d = to_dev(generate(w))
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    gam = dra.chunk_cumsum(d["g"])
    _, _, km, _, _ = dra.kda_prep(d["q"], d["k"], gam, flags=flags)
    torch.cuda.synchronize()
    mx = km.float().abs().max().item()
    emax = torch.exp2(-gam).max().item()
    print(f"stress: max|K-| = {mx:.1f}, max 2^-gamma = {emax:.1f}, flags = {flags.item()}", flush=True)
    assert np.isfinite(mx) and mx < 65504.0
    assert flags.item() == (1 if emax >= 65536.0 else 0)
