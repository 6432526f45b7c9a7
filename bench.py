#!/usr/bin/env python3
"""Benchmark of the chunkwise gated-delta-rule forward on one MI355X.

One step = one full forward pass (every step of the hot path: log2 cumsum,
separable prep and UT transform in the chunk-parallel kernel, then the
sequential state pass fused with the chunk output) over the KDA bf16
long-context workload (B=1, H=32, T=32768, dk=dv=128, C=64), inputs resident
in HBM.  Prints one JSON line.

Per-kernel durations come from HIP events recorded on the launch stream
between the two kernel launches of every timed step.  The step makes the same
two launches, on the same stream, as the kda_fwd entry point.  The HBM
traffic of each kernel comes from the committed counter summary under
profiles/ (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a copy-kernel
calibration); it is reported only while the kernel sources still hash to the
value recorded there.  The CPU baseline is the fp64 oracle (test
infrastructure) timed on a bounded sample of the same workload on the host
cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
METRIC = "fwd tokens/sec (1 GPU) for KDA/GDN chunked, bf16, T=32k; % MFMA peak"


def algorithmic(kind: str, w, io_bytes: int):
    """Bytes each kernel must move per token-head (its own inputs and
    outputs) and the method's MFMA flops per token-head (fixed formula)."""
    dk, dv, C = w.Dk, w.Dv, w.C
    delta = kind != "decay_la"
    gate = 4 * dk if kind == "kda" else 4
    beta = 4 if delta else 0
    # K1 reads q, k, v, g, beta; writes the chunk record: per row of the
    # chunk W (delta kinds only), Q~, Kbar^T, Aqk, U^T (V for decay_la), and
    # phi once per chunk
    rec_row = io_bytes * ((3 if delta else 2) * dk + C + dv) + 4 * dk / C
    k1 = io_bytes * (2 * dk + dv) + gate + beta + rec_row
    # K2 reads the record, writes o; h0/hT once per chain (negligible)
    k2 = rec_row + io_bytes * dv
    # per token-head MFMA flops of the method: KK^T, QK^T, W/U, A*Vnew, W*S,
    # Kbar^T*Vnew, Q*S and the inverse (full-tile count, fixed formula)
    if delta:
        flops = 2 * dk * C + 2 * dk * C + 2 * C * (dk + dv) + 2 * C * dv + 3 * 2 * dk * dv + 2 * C * C / 3
    else:
        flops = 2 * dk * C + 2 * C * dv + 2 * 2 * dk * dv
    return k1, k2, flops


def segment_plan(w):
    """(segments per chain, chunks per segment) as the library chooses them
    (about 256 workgroups for the segment kernel)."""
    NT = -(-w.T // w.C)
    chains = w.B * w.H
    if NT > 1 and chains < 256:
        want = min(NT, -(-256 // chains))
        L = -(-NT // want)
        return -(-NT // L), L
    return 1, max(NT, 1)


def segment_bytes(kind: str, w, io_bytes: int):
    """Algorithmic bytes per launch of the segment-parallel forward's three
    kernels: what each must read and write once.
      segment: q, k, v, g, beta in; o_local out; q_eff out for the chunks of
               segments after the first; per (chain, segment) [M | N] out
               (fp32, Dk x (Dk + Dv)).
      compose: [M | N] of the segments in; S_in (I/O dtype, Dk x Dv) of the
               segments after the first and hT (fp32) out.
      correct: q_eff and o in, o out for the chunks of segments after the
               first; S_in of those segments in."""
    dk, dv = w.Dk, w.Dv
    NS, L = segment_plan(w)
    NT = -(-w.T // w.C)
    chains = w.B * w.H
    th = w.B * w.T * w.H
    th_late = chains * min(w.T, max(0, w.T - L * w.C))     # token-heads of segments >= 1
    gate = 4 * dk if kind == "kda" else 4
    beta = 4 if kind != "decay_la" else 0
    seg = th * (io_bytes * (2 * dk + dv) + gate + beta + io_bytes * dv) + th_late * io_bytes * dk \
        + chains * NS * dk * (dk + dv) * 4
    comp = chains * NS * dk * (dk + dv) * 4 + chains * (NS - 1) * dk * dv * io_bytes + chains * dk * dv * 4
    corr = th_late * io_bytes * (dk + 2 * dv) + chains * (NS - 1) * dk * dv * io_bytes
    del NT
    return {"segment": seg, "compose": comp, "correct": corr}


# The sources the forward's kernels are compiled from (the segment-parallel
# path's and the record path's), and the build script with the compiler flags.
FORWARD_KERNEL_SOURCES = ("csrc/common.h", "csrc/intra.h", "csrc/inter.h", "csrc/seg.h", "csrc/k_seg.hip",
                          "build.py")


def kernel_source_hash() -> str:
    """sha256 over the forward kernels' sources and the build script, in name
    order (a change anywhere else, e.g. the backward, leaves it alone)."""
    pkg = os.path.join(ROOT, "delta_rule_rnn_amd")
    files = sorted(os.path.join(pkg, f) for f in FORWARD_KERNEL_SOURCES)
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, fpath: str = "segment"):
    """HBM bytes per launch of each kernel from the committed counter summary
    (profiles/<workload>_traffic.txt for the segment path,
    profiles/<workload>_records_traffic.txt for the record path), or {} when
    absent or taken on other kernel sources."""
    suffix = "" if fpath == "segment" else "_records"
    path = os.path.join(ROOT, "profiles", f"{workload}{suffix}_traffic.txt")
    if not os.path.exists(path):
        return {}
    text = open(path).read()
    m = re.search(r"^source_sha256:\s*([0-9a-f]{64})", text, re.M)
    if not m or m.group(1) != kernel_source_hash():
        return {}
    out = {}
    for name, b in re.findall(r"^traffic\s+(\w+):.*\bbytes=(\d+)", text, re.M):
        out[name] = int(b)
    return out


def cpu_baseline(w, x, max_tokens: int, threads: int):
    import oracle
    import torch
    Ts = min(w.T, max_tokens)
    sl = lambda t: None if t is None else t[:, :Ts].contiguous()
    h0 = None if x["h0"] is None else x["h0"].transpose(-1, -2).contiguous()
    args = [sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"])]
    t0 = time.perf_counter()
    oracle.recurrence(w.kind, *args, h0, nthreads=threads)
    dt = time.perf_counter() - t0
    del torch
    tokens = w.B * Ts
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{w.kind} B={w.B} H={w.H} first {Ts} of {w.T} tokens, fp64 token recurrence, "
                      f"{threads} threads, {dt:.2f} s wall", "cpu": cpu_model()}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"



def call_bytes(kind: str, w, io_b: int, tokens: int, chains: int, h0: bool, backward: bool = False) -> int:
    """The least HBM traffic of one whole call: every input read once and
    every output written once (the chunk records and the backward's other
    workspace arrays are the implementation's own and are not counted).
    Forward: q, k, v, g, beta in, o out, per chain h0 in (if given) and hT
    out.  Backward: the same inputs plus do, then dq, dk, dv, dg, dbeta out,
    per chain h0 (if given) and dhT in, dh0 out.  tokens counts tokens over
    all sequences (each with the workload's H heads); chains counts
    (sequence, head) pairs."""
    dk, dv = w.Dk, w.Dv
    gate = 4 * dk if kind == "kda" else 4
    beta = 4 if kind != "decay_la" else 0
    inputs = io_b * (2 * dk + dv) + gate + beta
    state = 4 * dk * dv
    if backward:
        per_th = inputs + io_b * dv + inputs
        per_chain = state * ((1 if h0 else 0) + 2)
    else:
        per_th = inputs + io_b * dv
        per_chain = state * ((1 if h0 else 0) + 1)
    return per_th * tokens * w.H + per_chain * chains


def whole_call_roofline(kernel: str, alg_bytes: int, avg_ms: float):
    """HBM roofline of a whole library call (several launches), from its
    least traffic and its average duration between HIP events on the launch
    stream."""
    gbs = alg_bytes / (avg_ms * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "avg_ms": round(avg_ms, 4),
            "alg_bytes": int(alg_bytes)}


def time_calls(call, steps: int, warmup: int):
    """(wall ms per call, average ms per call between HIP events recorded on
    torch's current stream, which is the stream the library launches on)."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t0 = time.perf_counter()
    for e in evs:
        e[0].record(stream)
        call()
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / steps
    return ms, sum(e[0].elapsed_time(e[1]) for e in evs) / steps


def cpu_threads(args) -> int:
    """Threads of the CPU oracle: every core this process may use (its
    affinity mask, bounded by OMP_NUM_THREADS where the host sets the job's
    CPU share that way)."""
    n = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return args.cpu_threads or n


def cpu_baseline_backward(kind, x, do, dhT, Ts: int):
    """The oracle's reverse sweep (fp64 numpy, one thread) over the first Ts
    tokens of every head of the first sequence; tokens/s of that sample."""
    from threadpoolctl import threadpool_limits
    from oracle.backward import recurrence_backward
    sl = lambda t: None if t is None else t[:1, :Ts].contiguous()
    h0 = None if x.get("h0") is None else x["h0"][:1].transpose(-1, -2).contiguous()
    dT = None if dhT is None else dhT[:1].transpose(-1, -2).contiguous()
    t0 = time.perf_counter()
    with threadpool_limits(1):
        recurrence_backward(kind, sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]), h0, sl(do), dT)
    dt = time.perf_counter() - t0
    H = x["q"].shape[2]
    return {"value": Ts / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{kind} H={H} first {Ts} tokens of one sequence, fp64 reverse sweep over tokens "
                      f"(numpy, 1 thread), {dt:.2f} s wall"}

def decode_bench(args):
    """Recurrent decode step: --decode-batch sequences x the workload's heads
    and head size, --decode-tokens new tokens each per call, the state
    resident in HBM and updated in place.  One JSON line; HBM roofline of the
    decode kernel from the state read + write and the token I/O."""
    import torch
    import delta_rule_rnn_amd as dra
    from delta_rule_rnn_amd.inputs import WORKLOADS, generate

    w0 = WORKLOADS[args.workload]
    w = w0.with_(name=w0.name + "_decode", B=args.decode_batch, T=args.decode_tokens, h0_std=0.5)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = generate(w)
    d = {n: (t.to(dev) if t is not None else None) for n, t in x.items()}
    state = d["h0"].clone()
    o = torch.empty(w.B, w.T, w.H, w.Dv, dtype=d["q"].dtype, device=dev)
    stream = torch.cuda.current_stream()
    call = lambda: dra.decode(w.kind, d["q"], d["k"], d["v"], d["g"], d["beta"], state, out=o)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in evs:
        e[0].record(stream)
        call()
        e[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1000.0 / args.steps
    k_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    io = 2 if d["q"].dtype == torch.bfloat16 else 4
    th = w.B * w.T * w.H
    per_chain = 2 * w.Dk * w.Dv * 4                      # state read + write
    per_token = io * (2 * w.Dk + 2 * w.Dv) + (4 * w.Dk if w.kind == "kda" else 4) + (4 if w.kind != "decay_la" else 0)
    alg = w.B * w.H * per_chain + th * per_token
    gbs = alg / (k_ms * 1e-3) / 1e9
    line = {
        "metric": "decode tokens/sec (1 GPU), recurrent step", "value": round(w.B * w.T / (ms / 1000.0), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if io == 2 else "f32", "data": "synthetic",
        "config": {"workload": f"{w.kind}_decode B={w.B} H={w.H} T={w.T} dk={w.Dk} dv={w.Dv}",
                   "global_batch": w.B, "seq_len": w.T, "heads": w.H, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "decode", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "avg_ms": round(k_ms, 4), "alg_bytes": int(alg)},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_decode(w, x, cpu_threads(args)),
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_decode(w, x, threads: int):
    """The oracle's token recurrence on the same decode call (every sequence,
    head and new token from the same states), repeated for about 2 s."""
    import oracle
    h0 = x["h0"].transpose(-1, -2).contiguous()
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.recurrence(w.kind, x["q"], x["k"], x["v"], x["g"], x["beta"], h0, nthreads=threads)
        n += 1
        dt = time.perf_counter() - t0
        if dt >= 2.0:
            break
    return {"value": n * w.B * w.T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole decode call ({w.B} sequences x {w.T} tokens, H={w.H}) {n} times, fp64 token "
                      f"recurrence, {threads} threads, {dt:.2f} s wall"}


def varlen_bench(args):
    """Forward over packed sequences: the workload's B*T tokens cut into
    sequences of seeded lengths uniform in [64, 4096] (the last one takes the
    remainder); same heads, head size and distributions as the workload."""
    import torch
    import delta_rule_rnn_amd as dra
    from delta_rule_rnn_amd.inputs import WORKLOADS, generate, packed_lengths

    w0 = WORKLOADS[args.workload]
    T = w0.B * w0.T
    w = w0.with_(name=w0.name + "_packed", B=1, T=T)
    lengths = packed_lengths(T, seed=7)
    cu = torch.tensor([0] + list(torch.tensor(lengths).cumsum(0).tolist()), dtype=torch.int32)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = generate(w)
    d = {n: (t.to(dev) if t is not None else None) for n, t in x.items()}
    sq = lambda t: None if t is None else t[0]
    cu = cu.to(dev)
    N = len(lengths)
    ws = torch.empty(dra.workspace_bytes_varlen(w.kind, N, T, w.H, w.Dk, w.Dv, d["q"].dtype), dtype=torch.uint8,
                     device=dev)
    call = lambda: dra.forward_varlen(w.kind, sq(d["q"]), sq(d["k"]), sq(d["v"]), sq(d["g"]), sq(d["beta"]), cu,
                                      workspace=ws)
    ms, ev_ms = time_calls(call, args.steps, args.warmup)
    io_b = 2 if d["q"].dtype == torch.bfloat16 else 4
    roof = whole_call_roofline("dr_forward_varlen (chunk table, K1, K2)",
                               call_bytes(w.kind, w, io_b, T, N * w.H, h0=False), ev_ms)
    cpu = None
    if not args.no_cpu_baseline:
        threads = cpu_threads(args)
        # whole sequences from the front of the batch, up to --cpu-tokens
        n, Ts = 0, 0
        while n < N and (n == 0 or Ts + lengths[n] <= args.cpu_tokens):
            Ts += lengths[n]
            n += 1
        import oracle
        t0 = time.perf_counter()
        a = 0
        for i in range(n):
            sl = lambda t: None if t is None else t[:, a:a + lengths[i]].contiguous()
            oracle.recurrence(w.kind, sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]), None,
                              nthreads=threads)
            a += lengths[i]
        dt = time.perf_counter() - t0
        cpu = {"value": Ts / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"the first {n} sequences ({Ts} tokens, H={w.H}), fp64 token recurrence, "
                         f"{threads} threads, {dt:.2f} s wall"}
    line = {
        "metric": "packed-sequence fwd tokens/sec (1 GPU)", "value": round(T / (ms / 1000.0), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if d["q"].dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": f"{w.kind}_fwd_varlen N={N} T={T} H={w.H} dk={w.Dk} dv={w.Dv} C={w.C}",
                   "sequences": N, "min_len": min(lengths), "max_len": max(lengths), "parallelism": "single GPU"},
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def backward_bench(args):
    """Backward of the workload's forward (dq, dk, dv, dg, dbeta, dh0 from do
    and dhT), inputs and cotangents resident in HBM, one dr_backward call per
    step timed with HIP events on the launch stream.  The split between its
    kernels comes from a rocprofv3 kernel trace (profiles/)."""
    import torch
    import delta_rule_rnn_amd as dra
    from delta_rule_rnn_amd.inputs import WORKLOADS, generate

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = generate(w)
    d = {n: (t.to(dev) if t is not None else None) for n, t in x.items()}
    gen = torch.Generator().manual_seed(99)
    do_c = torch.randn(w.B, w.T, w.H, w.Dv, generator=gen).to(d["q"].dtype)
    dhT_c = torch.randn(w.B, w.H, w.Dk, w.Dv, generator=gen) * 0.1
    do, dhT = do_c.to(dev), dhT_c.to(dev)
    ws = torch.empty(dra.backward_workspace_bytes(w.kind, w.B, w.T, w.H, w.Dk, w.Dv, d["q"].dtype),
                     dtype=torch.uint8, device=dev)
    call = lambda: dra.backward(w.kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], do, dhT, workspace=ws)
    ms, ev_ms = time_calls(call, args.steps, args.warmup)
    tokens = w.B * w.T
    io_b = 2 if d["q"].dtype == torch.bfloat16 else 4
    roof = whole_call_roofline("dr_backward (all launches)",
                               call_bytes(w.kind, w, io_b, tokens, w.B * w.H, h0=d["h0"] is not None,
                                          backward=True), ev_ms)
    cpu = None if args.no_cpu_baseline else cpu_baseline_backward(w.kind, x, do_c, dhT_c,
                                                                   min(w.T, args.cpu_bwd_tokens))
    line = {
        "metric": "bwd tokens/sec (1 GPU), all gradients", "value": round(tokens / (ms / 1000.0), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 compute, " + ("bf16" if d["q"].dtype == torch.bfloat16 else "f32") + " I/O",
        "data": "synthetic",
        "config": {"workload": f"{w.kind}_bwd B={w.B} H={w.H} T={w.T} dk={w.Dk} dv={w.Dv} C={w.C}",
                   "workspace_bytes": ws.numel(), "parallelism": "single GPU"},
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def backward_varlen_bench(args):
    """Backward over the packed batch of --mode varlen (the workload's B*T
    tokens in sequences of seeded lengths uniform in [64, 4096]), inputs,
    per-sequence initial states and cotangents resident in HBM, one
    dr_backward_varlen call per step."""
    import torch
    import delta_rule_rnn_amd as dra
    from delta_rule_rnn_amd.inputs import WORKLOADS, generate, packed_lengths

    w0 = WORKLOADS[args.workload]
    T = w0.B * w0.T
    w = w0.with_(name=w0.name + "_packed", B=1, T=T)
    lengths = packed_lengths(T, seed=7)
    N = len(lengths)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = generate(w)
    d = {n: (t.to(dev) if t is not None else None) for n, t in x.items()}
    sq = lambda t: None if t is None else t[0]
    cu = torch.tensor([0] + list(torch.tensor(lengths).cumsum(0).tolist()), dtype=torch.int32).to(dev)
    gen = torch.Generator().manual_seed(99)
    do_c = torch.randn(T, w.H, w.Dv, generator=gen).to(d["q"].dtype)
    dhT_c = torch.randn(N, w.H, w.Dk, w.Dv, generator=gen) * 0.1
    h0_c = torch.randn(N, w.H, w.Dk, w.Dv, generator=gen) * 0.1
    do, dhT, h0 = do_c.to(dev), dhT_c.to(dev), h0_c.to(dev)
    ws = torch.empty(dra.backward_varlen_workspace_bytes(w.kind, N, T, w.H, w.Dk, w.Dv, d["q"].dtype),
                     dtype=torch.uint8, device=dev)
    call = lambda: dra.backward_varlen(w.kind, sq(d["q"]), sq(d["k"]), sq(d["v"]), sq(d["g"]), sq(d["beta"]), cu,
                                       h0, do, dhT, workspace=ws)
    ms, ev_ms = time_calls(call, args.steps, args.warmup)
    io_b = 2 if d["q"].dtype == torch.bfloat16 else 4
    roof = whole_call_roofline("dr_backward_varlen (all launches)",
                               call_bytes(w.kind, w, io_b, T, N * w.H, h0=True, backward=True), ev_ms)
    cpu = None
    if not args.no_cpu_baseline:
        # a prefix of the first sequence is itself a sequence
        first = dict(x, h0=h0_c[:1])
        cpu = cpu_baseline_backward(w.kind, first, do_c.unsqueeze(0), dhT_c[:1],
                                    min(lengths[0], args.cpu_bwd_tokens))
    line = {
        "metric": "packed-sequence bwd tokens/sec (1 GPU), all gradients", "value": round(T / (ms / 1000.0), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 compute, " + ("bf16" if d["q"].dtype == torch.bfloat16 else "f32") + " I/O",
        "data": "synthetic",
        "config": {"workload": f"{w.kind}_bwd_varlen N={N} T={T} H={w.H} dk={w.Dk} dv={w.Dv} C={w.C}",
                   "sequences": N, "min_len": min(lengths), "max_len": max(lengths),
                   "workspace_bytes": ws.numel(), "parallelism": "single GPU"},
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def prologue_bench(args):
    """Forward with the fused input prologue on raw projections (the
    workload's sizes; q, k unnormalised, beta logits, and for scalar gates
    the gate input with per-head A_log, dt_bias), timed as whole calls.
    Beside it, the same forward after an unfused pre-pass in plain torch ops
    on the GPU (L2 norm, scale, sigmoid, gate), which the prologue replaces."""
    import torch
    import delta_rule_rnn_amd as dra
    from delta_rule_rnn_amd.inputs import WORKLOADS, generate_raw

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    raw = generate_raw(w)
    d = {n: (t.to(dev) if t is not None else None) for n, t in raw.items()}
    has_beta = w.kind != "decay_la"
    scale = w.Dk ** -0.5
    pro = dra.Prologue(qk_l2norm=True, scale=scale, beta_sigmoid=has_beta,
                       A_log=d["A_log"], dt_bias=d["dt_bias"])
    ws = dra.ops.alloc_workspace(w.kind, d["q"], d["v"], w.C)

    def fused():
        return dra.forward(w.kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], workspace=ws,
                           prologue=pro)

    def unfused():
        qf, kf = d["q"].float(), d["k"].float()
        q = (qf / torch.sqrt((qf * qf).sum(-1, keepdim=True) + 1e-6) * scale).to(d["q"].dtype)
        k = (kf / torch.sqrt((kf * kf).sum(-1, keepdim=True) + 1e-6)).to(d["k"].dtype)
        beta = torch.sigmoid(d["beta"]) if has_beta else None
        g = d["g"]
        if d["A_log"] is not None:
            g = -torch.exp(d["A_log"]) * torch.nn.functional.softplus(g + d["dt_bias"])
        return dra.forward(w.kind, q, k, d["v"], g, beta, d["h0"], workspace=ws)

    def timeit(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1000.0 / args.steps

    ms, ev_ms = time_calls(fused, args.steps, args.warmup)
    ms_unfused = timeit(unfused)
    tokens = w.B * w.T
    io_b = 2 if d["q"].dtype == torch.bfloat16 else 4
    roof = whole_call_roofline("dr_forward (prologue fused into the forward's chunk kernel; all launches)",
                               call_bytes(w.kind, w, io_b, tokens, w.B * w.H, h0=d["h0"] is not None), ev_ms)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        from oracle.prologue import apply
        threads = cpu_threads(args)
        # the numpy prologue dominates: half the forward's sample
        Ts = min(w.T, max(1, args.cpu_tokens // 2))
        sl = lambda t: None if t is None else t[:, :Ts].contiguous()
        t0 = time.perf_counter()
        q, k, g, beta = apply(w.kind, sl(raw["q"]), sl(raw["k"]), sl(raw["g"]), sl(raw["beta"]), qk_l2norm=True,
                              scale=scale, beta_sigmoid=has_beta, A_log=raw["A_log"], dt_bias=raw["dt_bias"])
        h0 = None if raw["h0"] is None else raw["h0"].transpose(-1, -2).contiguous()
        oracle.recurrence(w.kind, q, k, sl(raw["v"]), g, beta, h0, nthreads=threads)
        dt = time.perf_counter() - t0
        cpu = {"value": w.B * Ts / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{w.kind} B={w.B} H={w.H} first {Ts} of {w.T} tokens: fp64 prologue (numpy), then the "
                         f"fp64 token recurrence on {threads} threads, {dt:.2f} s wall"}
    line = {
        "metric": "fwd tokens/sec (1 GPU) with the fused input prologue", "value": round(tokens / (ms / 1000.0), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if d["q"].dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": f"{w.kind}_fwd+prologue B={w.B} H={w.H} T={w.T} dk={w.Dk} dv={w.Dv} C={w.C}",
                   "prologue": "qk_l2norm, scale dk^-1/2" + (", beta sigmoid" if has_beta else "")
                               + (", gate generation" if d["A_log"] is not None else ""),
                   "parallelism": "single GPU"},
        "unfused_prepass": {"ms_per_step": round(ms_unfused, 4),
                            "tokens_per_s": round(tokens / (ms_unfused / 1000.0), 1)},
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="kda_bf16_long")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gdn", action="store_true",
                    help="leave out the GDN workload that the KDA benchmark line carries in `extra`")
    ap.add_argument("--cpu-tokens", type=int, default=32768,
                    help="tokens of the workload the CPU oracle is timed on")
    ap.add_argument("--cpu-bwd-tokens", type=int, default=2048,
                    help="tokens of one sequence the CPU oracle's backward is timed on")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--mode", choices=("prefill", "decode", "varlen", "prologue", "backward", "backward_varlen"), default="prefill",
                    help="prefill: the chunked forward (the benchmark line); decode: the "
                         "recurrent step on a serving-sized batch; varlen: the forward over "
                         "packed sequences of mixed lengths with the workload's token count; "
                         "prologue: the forward with the fused input prologue on raw inputs; "
                         "backward: all gradients of the forward")
    ap.add_argument("--decode-batch", type=int, default=256,
                    help="sequences per decode call (256 x H=32 fp32 states = 537 MB, beyond the 256 MB "
                         "last-level cache)")
    ap.add_argument("--decode-tokens", type=int, default=1, help="new tokens per sequence per call")
    ap.add_argument("--path", choices=("segment", "records"), default="segment",
                    help="segment: the forward entry points' segment-parallel launches (the "
                         "benchmark line); records: the chunk-record path (chunk-parallel kernel, "
                         "then the sequential state pass) for comparison")
    ap.add_argument("--chunk", type=int, choices=(64, 128), default=0,
                    help="chunk size C (default: the workload's, 64).  C = 128 runs the record path "
                         "with 64-token sub-chunks (the segment-parallel path is built for C = 64)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (3 times): the "
                         "reference for scaling the HBM byte counters of a profile")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        n = args.copy_calibration
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on one GPU (each (batch, head) chain is sequential and no "
              "multi-GPU sharding is implemented); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.mode == "decode":
        decode_bench(args)
        return
    if args.mode == "varlen":
        varlen_bench(args)
        return
    if args.mode == "prologue":
        prologue_bench(args)
        return
    if args.mode == "backward":
        backward_bench(args)
        return
    if args.mode == "backward_varlen":
        backward_varlen_bench(args)
        return

    from delta_rule_rnn_amd.inputs import WORKLOADS

    w = WORKLOADS[args.workload]
    if args.chunk:
        w = w.with_(C=args.chunk)
    if w.C != 64:
        args.path = "records"
    r = time_forward(w, args.path, args.steps, args.warmup, args.workload)
    # the metric names KDA and GDN: the scalar-gate workload of the same
    # shape, timed the same way, rides along (not part of `value`)
    extra = {}
    if args.workload == "kda_bf16_long" and not args.no_gdn:
        wg = WORKLOADS["gdn_bf16_long"].with_(C=w.C)
        rg = time_forward(wg, args.path, args.steps, args.warmup, "gdn_bf16_long")
        extra["gdn_bf16_long"] = {"workload": rg["workload"], "value": rg["value"], "unit": "tokens/s",
                                  "ms_per_step": rg["ms"], "roofline": rg["roof"]}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, r["x"], args.cpu_tokens, cpu_threads(args))

    line = {
        "metric": METRIC, "value": r["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": r["dtype"], "data": "synthetic",
        "config": {"workload": r["workload"], "path": args.path,
                   "global_batch": w.B, "seq_len": w.T, "heads": w.H, "parallelism": "single GPU",
                   "gate": f"a ~ U[{w.gate_lo}, {w.gate_hi}]"},
        "median_ms_per_step_events": r["median_ev"],
        "min_ms_per_step_events": r["min_ev"],
        "mall_flushed": {"median_ms": r["cold_median"], "min_ms": r["cold_min"],
                         "note": "512 MB written before each step, outside its events"},
        "mfma_frac_bf16": r["mfma_frac"],
        "roofline": r["roof"],
        "cpu_baseline": cpu,
        "gate_flags": r["flags"],
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


def time_forward(w, path: str, steps: int, warmup: int, workload_name: str) -> dict:
    """One workload's forward on `path`: warmup, then `steps` timed steps
    (wall clock around all of them, HIP events per launch on the launch
    stream), then the same steps with the last-level cache flushed; the
    roofline of the dominant kernel."""
    import torch
    import delta_rule_rnn_amd as dra
    from delta_rule_rnn_amd import ops
    from delta_rule_rnn_amd.inputs import generate

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = generate(w)
    d = {n: (t.to(dev) if t is not None else None) for n, t in x.items()}
    B, T, H, Dk, Dv = w.B, w.T, w.H, w.Dk, w.Dv
    io = d["q"].dtype
    o = torch.empty(B, T, H, Dv, dtype=io, device=dev)
    hT = torch.empty(B, H, Dk, Dv, dtype=torch.float32, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    io_b = 2 if io == torch.bfloat16 else 4
    th = B * T * H
    if path == "segment":
        # the three launches of the forward entry points (dr_forward_stage
        # 0, 1, 2): local segment pass, entry-state composition, correction
        ws = ops.alloc_segment_workspace(w.kind, d["q"], d["v"], w.C)
        names = ("segment", "compose", "correct")

        def launches():
            yield lambda: dra.ops.forward_stage(0, w.kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"],
                                                out=o, workspace=ws, chunk_size=w.C, flags=flags)
            yield lambda: dra.ops.forward_stage(1, w.kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"],
                                                out=o, hT=hT, workspace=ws, chunk_size=w.C)
            yield lambda: dra.ops.forward_stage(2, w.kind, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"],
                                                out=o, workspace=ws, chunk_size=w.C)
        kbytes = segment_bytes(w.kind, w, io_b)
        flops = algorithmic(w.kind, w, io_b)[2]
    else:
        # the record path: chunk-parallel kernel, then the state pass
        ws = ops.alloc_record_workspace(w.kind, d["q"], d["v"], w.C)
        names = ("intra", "inter")

        def launches():
            yield lambda: dra.intra(w.kind, d["q"], d["k"], d["v"], d["g"], d["beta"], w.C, workspace=ws,
                                    flags=flags)
            yield lambda: dra.inter(w.kind, ws, B, T, H, Dk, Dv, io, h0=d["h0"], out=o, hT=hT, chunk_size=w.C)
        b1, b2, flops = algorithmic(w.kind, w, io_b)
        kbytes = {"intra": b1 * th, "inter": b2 * th}

    nl = len(names)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        for i, launch in enumerate(launches()):
            launch()
            if ev is not None:
                ev[i + 1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nl + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = {n: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / len(evs) for i, n in enumerate(names)}
    per_step = sorted(e[0].elapsed_time(e[nl]) for e in evs)

    # the same steps with the 256 MB last-level cache (MALL) flushed before
    # each one by a 512 MB write; only the step itself is inside the events
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(steps):
        flush.fill_(1)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(nl + 1)]
        step(ev)
        torch.cuda.synchronize()
        cold.append(ev[0].elapsed_time(ev[nl]))
    cold.sort()
    del flush
    ms = wall * 1000.0 / steps
    value = B * T / (ms / 1000.0)

    kern = {n: {"avg_ms": kms[n], "bytes": kbytes[n], "gbs": kbytes[n] / (kms[n] * 1e-3) / 1e9} for n in names}
    dom = max(kern, key=lambda n: kern[n]["avg_ms"])
    traffic = measured_traffic(workload_name + ("_c128" if w.C != 64 else ""), path)
    roof = {"bound": "hbm", "kernel": dom, "achieved": round(kern[dom]["gbs"], 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(kern[dom]["gbs"] / HBM_PEAK_GBS, 4),
            "traffic": traffic.get(dom),
            "per_kernel": {n: {"avg_ms": round(v["avg_ms"], 4), "alg_bytes": int(v["bytes"]),
                               "achieved_GBs": round(v["gbs"], 1), "traffic": traffic.get(n)}
                           for n, v in kern.items()}}
    mfma_frac = flops * th / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)
    return {"x": x, "value": round(value, 1), "ms": round(ms, 4), "roof": roof,
            "dtype": "bf16" if io == torch.bfloat16 else "f32",
            "workload": f"{w.kind}_fwd B={B} H={H} T={T} dk={Dk} dv={Dv} C={w.C}",
            "median_ev": round(per_step[len(per_step) // 2], 4), "min_ev": round(per_step[0], 4),
            "cold_median": round(cold[len(cold) // 2], 4), "cold_min": round(cold[0], 4),
            "mfma_frac": round(mfma_frac, 4), "flags": int(flags.item())}


if __name__ == "__main__":
    main()
