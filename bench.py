#!/usr/bin/env python3
"""Benchmark of the linear-attention hot path on one MI355X.

One step = one causal prefill call of a fresh sequence (la_causal_fwd_ws, the entry point with a
caller-owned workspace, from the zero state: phi on the loads, chunked matrix-core intra-chunk
product, carried float32 state, normaliser, bf16 store, final state S, z written) over the
workload B=2 H=16 N=8192
d=d_v=128 bf16, inputs IID N(0, 1/128). K steps are timed
between device synchronisations; input sets rotate over three copies (806 MB > the 256 MB
last-level cache) so a step does not find its inputs cached by the previous one.

Printed: one JSON line with the headline (token-heads per second); the HBM roofline of the
dominant kernel, k_causal, from HIP events the library records on the launch stream around each
of its kernels (la_causal_fwd_profiled), with the whole call's fraction beside it; the float64
oracle timed on the host; and the decode (B=256 H=32 d=128, 4096-token state) and global
(B=1 H=8 N=100000) forms.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
BF16_PEAK = 2.5e15         # flop/s, dense bf16 MFMA
FP32_MFMA_PEAK = 157.3e12  # flop/s, dense float32 MFMA
METRIC = "causal prefill tokens/s (B·H·N/s) at d=128 + %MFMA peak; decode step GB/s"


def algo_prefill(B, H, N, d, dv, es=2):
    """Algorithmic bytes and flops of one causal call: read q, k, v, write out, write the
    final float32 state; 4*d*dv + 3*d + dv flops per token-head."""
    th = B * H * N
    byts = th * ((2 * d + dv) * es + dv * es) + B * H * (d * dv + d) * 4
    flops = th * (4 * d * dv + 3 * d + dv)
    return byts, flops


def mfma_issued_prefill(B, H, N, P, d=128):
    """Matrix-core flops the chunked kernels issue (16x16x32 bf16 = 16384 flops each) for
    d = d_v = 128, chunk 64: per chunk 40 score + 48 intra + 128 state-read + 128 state-write
    instructions in the output kernel, and 128 in the segment-sum kernel for segments 0..P-2."""
    chunks = B * H * math.ceil(N / 64)
    per_chunk = 40 + 48 + 128 + 128 + 128 * (P - 1) / P
    return chunks * per_chunk * 16384


def mfma32_issued_prefill(B, H, N, P, d=128):
    """Matrix-core flops the float32 kernels issue (16x16x4 = 2048 flops each) for d = d_v,
    chunk 32: per token 4 d^2 (state read and state update) plus the three 16x16 score tiles and
    the twelve score-value products of a chunk per 16 value columns (48 (d + d_v) per token) in
    the output kernel, and 2 d^2 per token in the segment sums for segments 0..P-2."""
    th = B * H * N
    return th * (4 * d * d + 96 * d + 2 * d * d * (P - 1) / P)


def time_calls(fn, steps, warmup):
    """Average ms per call measured with HIP events on the current (launch) stream."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(st)
    for i in range(steps):
        fn(i)
    ev1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return ev0.elapsed_time(ev1) / steps, wall


def bench_prefill(args):
    import torch
    import causal_linear_attention_la_amd as la
    import datagen

    w = datagen.WORKLOADS[3]
    dev = torch.device("cuda:0")
    sets = []
    for r in range(args.rotate):
        q, k, v = datagen.qkv_cuda(w.B, w.H, w.N, w.d, w.dv, w.seed + 100 * r, w.scale, "bf16")
        out = torch.empty_like(q)
        S = torch.empty(w.B, w.H, w.d, w.dv, device=dev)
        z = torch.empty(w.B, w.H, w.d, device=dev)
        sets.append((q, k, v, out, S, z))

    # the segment-state workspace, owned by the caller and shared by the steps (one stream)
    need = la.la_workspace_bytes(0, w.B, w.H, w.N, w.d, w.dv, args.chunk, args.seg_len)
    ws = torch.empty(max(need, 16) // 4, dtype=torch.float32, device=dev)

    def step(i):
        # a fresh sequence: zero initial state (no buffer), final state written to S, z
        q, k, v, out, S, z = sets[i % len(sets)]
        la.la_causal_fwd_ws(q, k, v, out, ws if need else None, None, None, S, z,
                            chunk=args.chunk, seg_len=args.seg_len)

    # The same call in the chip's steady state first (200 untimed calls, then 200 timed), reported
    # on its own: measured on MI355X, the first few hundred calls of a process run 3-15 % slower
    # than the sustained rate (calls 5-25 at 95-97 us, 25-100 at 98-107 us, 300-400 at 92 us), so
    # the headline's own W warm-up and K timed steps follow it.
    ms_steady = time_calls(step, args.steady, args.steady)[0] if args.steady else None
    ms, wall = time_calls(step, args.steps, args.warmup)
    # same buffers every step (inputs may stay in the last-level cache)
    ms_hot, _ = time_calls(lambda i: step(0), args.steps, 2)

    # per-kernel device times: HIP events recorded by the library on the launch stream around
    # each kernel of `steps` back-to-back calls (segment sums, the scan where one is launched,
    # causal outputs)
    q, k, v, out, S, z = sets[0]
    la.la_causal_fwd_profiled(q, k, v, out, None, None, S, z, chunk=args.chunk,
                              seg_len=args.seg_len, reps=2)
    kern_ms = list(la.la_causal_fwd_profiled(q, k, v, out, None, None, S, z, chunk=args.chunk,
                                             seg_len=args.seg_len, reps=args.steps))
    byts, flops = algo_prefill(w.B, w.H, w.N, w.d, w.dv)
    # segments per head the library chose
    P = la.la_segments(0, w.B, w.H, w.N, w.d, w.dv, args.chunk, args.seg_len)
    return w, ms, ms_hot, wall, byts, flops, P, kern_ms, ms_steady


def kernels_us(kern, P, scan):
    """Per-kernel device times (us) of one causal call from la_causal_fwd_profiled: the segment
    sums, the scan over segment states (launched on the float32 and vector-ALU paths only: on
    the bf16 matrix-core path each causal segment adds up the sums before it itself) and the
    causal kernel; with one segment the causal kernel alone."""
    if P <= 1:
        return {"causal": kern[2] * 1e3}
    out = {"segment_sums": kern[0] * 1e3}
    if scan:
        out["segment_scan"] = kern[1] * 1e3
    out["causal"] = kern[2] * 1e3
    return out


def time_flushed(fn, reps, flush_bytes=512 << 20):
    """Average device ms of fn() when each call starts with none of its data in the caches:
    before every call a 512 MiB buffer (twice the 256 MB last-level cache) is read through, and
    only the call itself is timed, between HIP events on the launch stream."""
    import torch
    buf = torch.ones(flush_bytes // 4, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    fn()
    torch.cuda.synchronize()
    for a, b in evs:
        buf.max()
        a.record(st)
        fn()
        b.record(st)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / reps


GRAPH_CALLS = 20


def bench_causal_small(args, n):
    """Causal workloads 1 (B=1 H=1 N=64 d=16 float32, the vector-ALU kernels) and 2 (B=4 H=8
    N=2048 d=64 bf16, chunk 64: the d = 64 matrix-core kernels), through la_causal_fwd_ws from
    the zero state with the final state written. Both are small enough to sit in the caches, so
    they are timed hot (the same buffers back to back) and flushed (time_flushed); for workload
    2 the per-kernel times come from the library's own HIP events (la_causal_fwd_profiled)."""
    import torch
    import causal_linear_attention_la_amd as la
    import datagen

    w = datagen.WORKLOADS[n]
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in datagen.qkv(w.B, w.H, w.N, w.d, w.dv, w.seed, w.scale, w.dtype))
    out = torch.empty_like(v)
    S = torch.empty(w.B, w.H, w.d, w.dv, device=dev)
    z = torch.empty(w.B, w.H, w.d, device=dev)
    code = la.LA_BF16 if w.dtype == "bf16" else la.LA_F32
    need = la.la_workspace_bytes(0, w.B, w.H, w.N, w.d, w.dv, w.chunk, 0, code)
    ws = torch.empty(max(need, 16) // 4, dtype=torch.float32, device=dev) if need else None

    def call(i=0):
        la.la_causal_fwd_ws(q, k, v, out, ws, None, None, S, z, chunk=w.chunk)

    ms_hot, _ = time_calls(call, args.steps, args.warmup)
    ms_flushed = time_flushed(call, max(10, args.steps // 4))
    # the same call replayed from a HIP graph (GRAPH_CALLS calls per graph, kernel nodes only):
    # the device time per call without the host's per-call cost (argument checks, launch),
    # which a call this small is otherwise bound by
    graph = torch.cuda.CUDAGraph()
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(gs):
        with torch.cuda.graph(graph, stream=gs):
            for _ in range(GRAPH_CALLS):
                call()
    torch.cuda.synchronize()
    ms_graph = time_calls(lambda i: graph.replay(), max(10, args.steps // 2), 2)[0] / GRAPH_CALLS
    kern = la.la_causal_fwd_profiled(q, k, v, out, None, None, S, z, chunk=w.chunk,
                                     reps=args.steps)
    P = la.la_segments(0, w.B, w.H, w.N, w.d, w.dv, w.chunk, 0, code)
    return w, ms_hot, ms_flushed, ms_graph, kern, P


def bench_decode(args):
    import torch
    import causal_linear_attention_la_amd as la
    import datagen

    w = datagen.WORKLOADS[5]
    dev = torch.device("cuda:0")
    S = torch.empty(w.B, w.H, w.d, w.dv, device=dev)
    z = torch.empty(w.B, w.H, w.d, device=dev)
    # starting state: sums of phi(k) v^T over a 4096-token seeded prior, built with the
    # library's global form (state only) in blocks of batch rows
    for b0 in range(0, w.B, datagen.DECODE_PRIOR_BLOCK):
        kp, vp = datagen.decode_prior(w, b0)
        la.la_global_fwd(None, kp, vp, None, S[b0:b0 + kp.shape[0]], z[b0:b0 + kp.shape[0]])
        del kp, vp
    steps = args.decode_steps
    # fresh q, k, v for every step, drawn up front as [steps, B, H, d]
    toks = datagen.decode_tokens(w, steps)
    out = torch.empty(w.B, w.H, w.dv, dtype=torch.bfloat16, device=dev)

    def step(i):
        la.la_decode_step(toks[0][i % steps], toks[1][i % steps], toks[2][i % steps], out, S, z)

    ms, _ = time_calls(step, steps, 0)
    heads = w.B * w.H
    byts = heads * (2 * (w.d * w.dv + w.d) * 4 + (2 * w.d + w.dv) * 2 + w.dv * 2)
    return w, ms, byts


def bench_global(args):
    import torch
    import causal_linear_attention_la_amd as la
    import datagen

    w = datagen.WORKLOADS[4]
    dev = torch.device("cuda:0")
    q, k, v = datagen.qkv_cuda(w.B, w.H, w.N, w.d, w.dv, w.seed, w.scale, "bf16")
    out = torch.empty_like(q)
    S = torch.empty(w.B, w.H, w.d, w.dv, device=dev)
    z = torch.empty(w.B, w.H, w.d, device=dev)
    ms, _ = time_calls(lambda i: la.la_global_fwd(q, k, v, out, S, z), max(5, args.steps // 2), 2)
    th = w.B * w.H * w.N
    byts = th * (4 * w.d * 2) + w.B * w.H * (w.d * w.dv + w.d) * 4
    return w, ms, byts


def bench_favor(args):
    """Positive random features (m = 128 projections) on the prefill workload's inputs: the
    one-call form la_causal_fwd_rf (the map runs inside the attention kernels' staging), and
    the two-pass form (la_rf_features on q and on k, then la_causal_fwd_ex with
    LA_PHI_IDENTITY) beside it. Returns per-step and per-kernel times."""
    import torch
    import causal_linear_attention_la_amd as la
    import datagen

    rw = datagen.RF_WORKLOAD
    w = datagen.WORKLOADS[rw["base"]]
    m = rw["m"]
    dev = torch.device("cuda:0")
    W = datagen.projections(m, w.d, rw["seed"], "bf16").to(dev)
    sets = []
    for r in range(args.rotate):
        q, k, v = datagen.qkv_cuda(w.B, w.H, w.N, w.d, w.dv, w.seed + 100 * r, w.scale, "bf16")
        fq = torch.empty((w.B, w.H, w.N, m), dtype=torch.bfloat16, device=dev)
        fk = torch.empty_like(fq)
        out = torch.empty_like(v)
        S = torch.empty(w.B, w.H, m, w.dv, device=dev)
        z = torch.empty(w.B, w.H, m, device=dev)
        sets.append((q, k, v, fq, fk, out, S, z))

    def step(i):
        q, k, v, fq, fk, out, S, z = sets[i % len(sets)]
        la.la_causal_fwd_rf(q, k, v, out, W, None, None, S, z)

    def two_pass(i):
        q, k, v, fq, fk, out, S, z = sets[i % len(sets)]
        la.la_rf_features(q, W, fq)
        la.la_rf_features(k, W, fk)
        la.la_causal_fwd_ex(fq, fk, v, out, None, None, S, z, flags=la.LA_PHI_IDENTITY)

    ms, _ = time_calls(step, args.steps, args.warmup)
    ms_two, _ = time_calls(two_pass, args.steps, 2)

    def rf_only(i):
        q, _, _, fq, _, _, _, _ = sets[i % len(sets)]
        la.la_rf_features(q, W, fq)

    ms_rf, _ = time_calls(rf_only, args.steps, 2)
    q, k, v, fq, fk, out, S, z = sets[0]
    kern = la.la_causal_fwd_profiled(fq, fk, v, out, None, None, S, z, flags=la.LA_PHI_IDENTITY,
                                     reps=args.steps)
    rows = w.B * w.H * w.N
    rf_bytes = rows * (w.d + m) * 2 + m * w.d * 2
    return w, m, ms, ms_rf, rf_bytes, kern, ms_two


def retention_name():
    import datagen
    return datagen.DECAY_WORKLOAD["name"]


def favor_name():
    import datagen
    return datagen.RF_WORKLOAD["name"]


def bench_variants(args):
    """Causal prefill with q, k taken as features and no division (LA_PHI_IDENTITY |
    LA_UNNORMALIZED) on the prefill workload: the cost of the form without phi and z."""
    import torch
    import causal_linear_attention_la_amd as la
    import datagen

    w = datagen.WORKLOADS[3]
    dev = torch.device("cuda:0")
    sets = []
    for r in range(args.rotate):
        q, k, v = datagen.qkv_cuda(w.B, w.H, w.N, w.d, w.dv, w.seed + 100 * r, w.scale, "bf16")
        out = torch.empty_like(q)
        S = torch.empty(w.B, w.H, w.d, w.dv, device=dev)
        z = torch.empty(w.B, w.H, w.d, device=dev)
        sets.append((q, k, v, out, S, z))
    flags = la.LA_PHI_IDENTITY | la.LA_UNNORMALIZED

    def step(i):
        q, k, v, out, S, z = sets[i % len(sets)]
        la.la_causal_fwd_ex(q, k, v, out, None, None, S, z, flags=flags)

    ms, _ = time_calls(step, args.steps, args.warmup)
    return w, ms


def bench_f32(args):
    """The prefill workload's shape in float32 (its inputs drawn in float32), through the
    workspace entry point: the float32 matrix-core kernels."""
    import torch
    import causal_linear_attention_la_amd as la
    import datagen

    w = datagen.WORKLOADS[3]
    dev = torch.device("cuda:0")
    sets = []
    for r in range(2):
        q, k, v = datagen.qkv_cuda(w.B, w.H, w.N, w.d, w.dv, w.seed + 100 * r, w.scale, "f32")
        sets.append((q, k, v, torch.empty_like(q), torch.empty(w.B, w.H, w.d, w.dv, device=dev),
                     torch.empty(w.B, w.H, w.d, device=dev)))
    need = la.la_workspace_bytes(0, w.B, w.H, w.N, w.d, w.dv, 0, 0, la.LA_F32)
    ws = torch.empty(max(need, 16) // 4, dtype=torch.float32, device=dev)

    def step(i):
        q, k, v, out, S, z = sets[i % len(sets)]
        la.la_causal_fwd_ws(q, k, v, out, ws if need else None, None, None, S, z)

    steps = max(20, args.steps // 4)
    ms, _ = time_calls(step, steps, max(5, args.warmup // 4))
    q, k, v, out, S, z = sets[0]
    kern_ms = list(la.la_causal_fwd_profiled(q, k, v, out, None, None, S, z, reps=steps))
    P = la.la_segments(0, w.B, w.H, w.N, w.d, w.dv, 0, 0, la.LA_F32)
    return w, ms, kern_ms, P


def bench_retention(args):
    """The decayed recurrence in its retention form (LA_PHI_IDENTITY | LA_UNNORMALIZED, per-head
    gamma = 1 - 2^-(5+h)) on the prefill workload's inputs: la_causal_fwd_decay per step."""
    import torch
    import causal_linear_attention_la_amd as la
    import datagen

    w = datagen.WORKLOADS[datagen.DECAY_WORKLOAD["base"]]
    dev = torch.device("cuda:0")
    gamma = datagen.decay_rates(w.H).to(dev)
    sets = []
    for r in range(args.rotate):
        q, k, v = datagen.qkv_cuda(w.B, w.H, w.N, w.d, w.dv, w.seed + 100 * r, w.scale, "bf16")
        out = torch.empty_like(q)
        S = torch.empty(w.B, w.H, w.d, w.dv, device=dev)
        z = torch.empty(w.B, w.H, w.d, device=dev)
        sets.append((q, k, v, out, S, z))
    flags = la.LA_PHI_IDENTITY | la.LA_UNNORMALIZED

    def step(i):
        q, k, v, out, S, z = sets[i % len(sets)]
        la.la_causal_fwd_decay(q, k, v, out, gamma, None, None, S, z, flags=flags)

    ms, _ = time_calls(step, args.steps, args.warmup)
    return w, ms


def bench_serving(args):
    """Prefill then decode for the same sequences: la_causal_fwd_state over an N-token prompt
    (B=2 H=16 N=8192 d=128) writes S, z; then K decode steps (la_decode_step, one token per
    sequence per step) continue from that state. The K steps are captured once in a HIP graph
    and replayed (no per-step launch from Python). One serving step = prefill + K decode
    steps; throughput counts prompt and generated tokens (per sequence, times heads)."""
    import torch
    import causal_linear_attention_la_amd as la
    import datagen

    w = datagen.WORKLOADS[3]
    K = args.serve_steps
    dev = torch.device("cuda:0")
    q, k, v = datagen.qkv_cuda(w.B, w.H, w.N, w.d, w.dv, w.seed, w.scale, "bf16")
    out = torch.empty_like(q)
    S = torch.empty(w.B, w.H, w.d, w.dv, device=dev)
    z = torch.empty(w.B, w.H, w.d, device=dev)
    toks = datagen.qkv_cuda(K, w.B * w.H, 1, w.d, w.dv, w.seed + 7, w.scale, "bf16")
    toks = [x.view(K, w.B, w.H, -1) for x in toks]
    dout = torch.empty(K, w.B, w.H, w.dv, dtype=torch.bfloat16, device=dev)

    def decode_all():
        for t in range(K):
            la.la_decode_step(toks[0][t], toks[1][t], toks[2][t], dout[t], S, z)

    # capture on a side stream (the library launches on the current stream)
    la.la_causal_fwd_state(q, k, v, out, None, None, S, z)
    decode_all()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode_all()
    torch.cuda.synchronize()

    def step(i):
        la.la_causal_fwd_state(q, k, v, out, None, None, S, z)
        graph.replay()

    ms, _ = time_calls(step, max(3, args.steps // 5), 2)
    ms_pre, _ = time_calls(lambda i: la.la_causal_fwd_state(q, k, v, out, None, None, S, z),
                           max(3, args.steps // 5), 1)
    return w, K, ms, ms_pre


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _median_runs(fn, seconds, at_least=3):
    times = []
    while len(times) < at_least or sum(times) < seconds:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return statistics.median(times), len(times)


def _single_thread(fn, seconds, at_least=2):
    """_median_runs of fn with the oracle on one host thread."""
    import oracle

    prev = oracle.set_threads(1)
    try:
        return _median_runs(fn, seconds, at_least)
    finally:
        oracle.set_threads(prev)


def cpu_baseline_causal(n, seconds=5.0):
    """The float64 oracle, as it stands, on causal workload n (the whole workload), on all host
    threads: median of repeated runs; and on at most 4 of its heads on one thread."""
    import datagen
    import oracle

    w = datagen.WORKLOADS[n]
    q, k, v = (datagen.to_f64(x) for x in datagen.qkv(w.B, w.H, w.N, w.d, w.dv, w.seed, w.scale,
                                                       w.dtype))
    t, runs = _median_runs(lambda: oracle.causal(q, k, v), seconds)
    h1 = min(4, w.H)
    t1, runs1 = _single_thread(lambda: oracle.causal(q[:1, :h1], k[:1, :h1], v[:1, :h1]), seconds / 2)
    return {"value": w.B * w.H * w.N / t, "unit": "tokens/s (B*H*N/s)", "cores": oracle.threads(),
            "kind": "oracle", "us_per_call": t * 1e6,
            "sample": f"{w.name}, the whole workload, float64 token-serial recurrence, median of "
                      f"{runs} runs of {t * 1e3:.2f} ms",
            "single_thread": {"value": h1 * w.N / t1, "unit": "tokens/s (B*H*N/s)", "cores": 1,
                              "sample": f"{h1} of the {w.B * w.H} heads, median of {runs1} runs of "
                                        f"{t1 * 1e3:.2f} ms"}}


def cpu_baseline_global(seconds=10.0):
    """The float64 oracle on the global workload (B=1 H=8 N=100000 d=128, the whole workload:
    state from every key, then every query read); its 8 heads split over the host threads."""
    import datagen
    import oracle

    w = datagen.WORKLOADS[4]
    q, k, v = (datagen.to_f64(x) for x in datagen.qkv_cuda(w.B, w.H, w.N, w.d, w.dv, w.seed,
                                                            w.scale, "bf16"))
    t, runs = _median_runs(lambda: oracle.global_(q, k, v), seconds, at_least=2)
    t1, runs1 = _single_thread(lambda: oracle.global_(q[:1, :1], k[:1, :1], v[:1, :1]), seconds / 2)
    return {"value": w.B * w.H * w.N / t, "unit": "tokens/s (B*H*N/s)", "cores": oracle.threads(),
            "kind": "oracle", "us_per_call": t * 1e6,
            "sample": f"{w.name}, the whole workload (inputs drawn on the device as the GPU leg "
                      f"does), float64, median of {runs} runs of {t:.2f} s; 8 heads, so at most 8 "
                      "threads have work",
            "single_thread": {"value": w.N / t1, "unit": "tokens/s (B*H*N/s)", "cores": 1,
                              "sample": f"1 of the {w.B * w.H} heads, median of {runs1} runs of "
                                        f"{t1:.2f} s"}}


def cpu_baseline_decode(seconds=10.0):
    """The float64 oracle's decode step on all 256 x 32 heads of the decode workload: steps per
    second over a few consecutive steps. The state is a seeded synthetic one of the decode
    state's shape and magnitude (building the 4096-token prior takes the oracle minutes; the
    time of a step does not depend on the values), the step tokens are the workload's."""
    import datagen
    import oracle

    w = datagen.WORKLOADS[5]
    S = datagen.to_f64(datagen.normal_cuda((w.B, w.H, w.d, w.dv), w.seed + 7, 6.0))
    z = 4096.0 + datagen.to_f64(datagen.normal_cuda((w.B, w.H, w.d), w.seed + 8, 64.0))
    nsteps = 4
    toks = [datagen.to_f64(x[:nsteps]) for x in datagen.decode_tokens(w, nsteps)]
    state = {"S": S, "z": z}

    def run():
        Sc, zc = state["S"], state["z"]
        for t in range(nsteps):
            _, Sc, zc = oracle.decode_step(toks[0][t], toks[1][t], toks[2][t], Sc, zc)

    t, runs = _median_runs(run, seconds, at_least=2)
    # one thread: the same steps over the first 16 of the 256 batch entries (512 heads), scaled
    # to all heads
    b1 = 16
    sub = {"S": state["S"][:b1], "z": state["z"][:b1]}

    def run1():
        Sc, zc = sub["S"], sub["z"]
        for t_ in range(nsteps):
            _, Sc, zc = oracle.decode_step(toks[0][t_][:b1], toks[1][t_][:b1], toks[2][t_][:b1], Sc, zc)

    t1, runs1 = _single_thread(run1, seconds / 3)
    scale = w.B / b1
    return {"value": nsteps / t, "unit": "decode steps/s (all 8192 heads per step)",
            "cores": oracle.threads(), "kind": "oracle", "us_per_step": t / nsteps * 1e6,
            "sample": f"{nsteps} consecutive decode steps of {w.name} from a seeded synthetic "
                      f"float64 state, median of {runs} runs of {t:.2f} s",
            "single_thread": {"value": nsteps / (t1 * scale),
                              "unit": "decode steps/s (all 8192 heads per step)", "cores": 1,
                              "sample": f"{nsteps} steps over {b1 * w.H} of the {w.B * w.H} heads, "
                                        f"median of {runs1} runs of {t1:.2f} s, scaled by {scale:g}"}}


def cpu_baseline():
    """The float64 oracle, as it stands, on the prefill workload's 32 heads (full size) on all
    host threads, and on 4 of its heads single-threaded: each repeated for about 10 s and 5 s
    of wall-clock time (at least 3 runs), median run."""
    import datagen
    import oracle

    w = datagen.WORKLOADS[3]
    heads = w.B * w.H
    q, k, v = datagen.qkv(w.B, w.H, w.N, w.d, w.dv, w.seed, w.scale, "bf16")
    qd, kd, vd = (datagen.to_f64(x) for x in (q, k, v))

    def med(fn, seconds):
        times = []
        while len(times) < 3 or sum(times) < seconds:
            t0 = time.perf_counter()
            fn()
            times.append(time.perf_counter() - t0)
        return statistics.median(times), len(times)

    t, n = med(lambda: oracle.causal(qd, kd, vd), 10.0)
    cores = oracle.threads()
    prev = oracle.set_threads(1)
    try:
        t1, n1 = med(lambda: oracle.causal(qd[:1, :4], kd[:1, :4], vd[:1, :4]), 5.0)
    finally:
        oracle.set_threads(prev)
    return {"value": w.B * w.H * w.N / t, "unit": "tokens/s (B*H*N/s)", "cores": cores,
            "kind": "oracle",
            "sample": f"causal B={w.B} H={w.H} N={w.N} d=128 ({heads} heads, the whole workload), "
                      f"float64 token-serial recurrence, median of {n} runs of {t:.2f} s",
            "single_thread": {"value": 4 * w.N / t1, "unit": "tokens/s (B*H*N/s)", "cores": 1,
                              "sample": f"4 of the {heads} heads, median of {n1} runs of {t1:.2f} s"},
            "host_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}


def copy_bandwidth(nbytes=256 << 20, reps=20):
    """Read + write bandwidth of a plain elementwise copy (dst = src * 1, float32) of `nbytes`
    on the box: the practical streaming rate the HBM-bound kernels are compared with."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = [torch.empty_like(src) for _ in range(2)]
    ms, _ = time_calls(lambda i: torch.mul(src, 1.0, out=dst[i % 2]), reps, 3)
    return 2 * nbytes / (ms * 1e-3)


def d2d_bandwidth(nbytes=205 << 20, reps=20):
    """Read + write bandwidth of a device-to-device copy (hipMemcpyAsync through tensor.copy_) of
    `nbytes` of varied bf16 data: the rate of a plain mixed read/write stream, which the causal
    kernel (218 MB read, 69 MB written per launch) is."""
    import torch
    n = nbytes // 2
    src = (torch.arange(n, device="cuda", dtype=torch.int32) * 40503).to(torch.int16).view(torch.bfloat16)
    dst = torch.empty_like(src)
    ms, _ = time_calls(lambda i: dst.copy_(src), reps, 3)
    return 2 * nbytes / (ms * 1e-3)


def rmw_bandwidth(nbytes, reps=10):
    """Read + write bandwidth of an in-place read-modify-write (x *= 1, float32) over `nbytes`:
    the pattern of a decode step, which reads and rewrites its state in place."""
    import torch
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    ms, _ = time_calls(lambda i: x.mul_(1.0), reps, 3)
    del x
    return 2 * nbytes / (ms * 1e-3)


def copy_calibration(nbytes=256 << 20, reps=5):
    """A plain elementwise copy kernel of known size (dst = src * 1, float32), for scaling the
    HBM byte counters FETCH_SIZE and WRITE_SIZE: each launch reads and writes nbytes."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    return nbytes


TRAFFIC_SOURCES = ("causal_linear_attention_la_amd/csrc/k_mfma.hip",
                   "causal_linear_attention_la_amd/csrc/la_api.hip")


def sources_digest():
    """SHA-256 over the code of the sources that decide the causal kernel's memory traffic (the
    kernel and the launch plan that sizes its segments): // comments, trailing blanks and empty
    lines are dropped first, so an edit of the comments keeps a measurement valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            for line in f:
                code = re.sub(r"//.*", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per launch of the causal kernel as last measured with rocprofv3 counters
    (profiles/k_causal_b2h16n8192_d128_traffic.json), or None when the kernel or its launch plan
    has changed since (the file stores the digest of the sources it was measured with)."""
    path = os.path.join(ROOT, "profiles", "k_causal_b2h16n8192_d128_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("sources_sha256") != sources_digest():
        return None
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 200 untimed then 200 timed calls of ~0.1 ms each: the figures are the chip's steady state
    # under continuous work (measured on MI355X, the same prefill call: 103 us per call in a
    # 50-call run after 5 warm-up calls, 97 us in 200 calls after 20, 92 us in 200 calls after
    # 200, 91 us after 500; the per-kernel times settle within the first ~50 calls)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--steady", type=int, default=200,
                    help="untimed and then timed calls of the prefill's steady-state leg, run "
                         "before the headline's W/K steps (0: skip)")
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--seg-len", dest="seg_len", type=int, default=0)
    ap.add_argument("--rotate", type=int, default=3, help="input sets cycled over the steps")
    ap.add_argument("--decode-steps", dest="decode_steps", type=int, default=1000)
    ap.add_argument("--serve-steps", dest="serve_steps", type=int, default=256,
                    help="decode steps after the prefill in the serving leg")
    ap.add_argument("--only", choices=["prefill", "decode", "global", "favor", "variants", "f32",
                                       "retention", "serving", "copycal", "small"],
                    default=None,
                    help="run one form only (for profiling); no JSON line")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copycal", action="store_true",
                    help="with --only: run the copy calibration kernel first (counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the heads of this "
              "workload are independent, so across GPUs each would take a slice of the B*H "
              "heads with no communication", file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.init()

    if args.only == "copycal":
        n = copy_calibration()
        print(f"copycal: copied {n} bytes x 5", flush=True)
        return
    if args.only == "small":
        if args.copycal:
            copy_calibration()
        for n in (1, 2):
            wn, hot, flushed, graph_ms, kern_n, _ = bench_causal_small(args, n)
            print(f"workload {n} ({wn.name}): hot {hot * 1e3:.1f} us, flushed {flushed * 1e3:.1f} us, "
                  f"graph-replayed {graph_ms * 1e3:.1f} us", flush=True)
        return
    if args.only:
        if args.copycal:
            copy_calibration()
        fn = {"prefill": bench_prefill, "decode": bench_decode, "global": bench_global,
              "favor": bench_favor, "variants": bench_variants, "retention": bench_retention,
              "f32": bench_f32,
              "serving": bench_serving}[args.only]
        r = fn(args)
        extra = ""
        if args.only == "prefill":
            extra = " (kernels: " + ", ".join(f"{t * 1e3:.1f}" for t in r[7]) + " us)"
        if args.only == "f32":
            extra = " (kernels: " + ", ".join(f"{t * 1e3:.1f}" for t in r[2]) + " us)"
        if args.only == "favor":
            extra = f" (two-pass {r[6] * 1e3:.1f} us: features {r[3] * 1e3:.1f} us per tensor; " + \
                "attention kernels " + ", ".join(f"{t * 1e3:.1f}" for t in r[5]) + " us)"
        ms = r[2] if args.only in ("favor", "serving") else r[1]
        print(f"{args.only}: {ms:.4f} ms/step{extra}", flush=True)
        return

    # The other forms run first: by the time the headline's own warm-up and timed steps run, the
    # chip has worked for several seconds and runs at its sustained clock (on a cold chip the
    # first few hundred calls run several percent slower while it ramps up).
    wd, ms_d, byts_d = bench_decode(args)
    # reference for the decode step: an in-place read-modify-write over a buffer of its state's
    # size (S and z in float32, 541 MB for the decode workload)
    rmw_bw = rmw_bandwidth(wd.B * wd.H * (wd.d * wd.dv + wd.d) * 4)
    print(f"decode: {ms_d * 1e3:.1f} us/step", file=sys.stderr, flush=True)
    wg, ms_g, byts_g = bench_global(args)
    print(f"global: {ms_g * 1e3:.1f} us/call", file=sys.stderr, flush=True)
    wf, m_f, ms_f, ms_rf, rf_bytes, kern_f, ms_f2 = bench_favor(args)
    print(f"favor: {ms_f * 1e3:.1f} us/step in one call, {ms_f2 * 1e3:.1f} us two-pass "
          f"(features {ms_rf * 1e3:.1f} us per tensor)", file=sys.stderr, flush=True)
    wv, ms_v = bench_variants(args)
    print(f"identity+unnormalised causal: {ms_v * 1e3:.1f} us/call", file=sys.stderr, flush=True)
    wr, ms_r = bench_retention(args)
    print(f"retention causal: {ms_r * 1e3:.1f} us/call", file=sys.stderr, flush=True)
    w32, ms_32, kern_32, P_32 = bench_f32(args)
    print(f"float32 causal: {ms_32 * 1e3:.1f} us/call; kernels "
          + ", ".join(f"{t * 1e3:.1f}" for t in kern_32) + " us", file=sys.stderr, flush=True)
    ws_, K_s, ms_s, ms_sp = bench_serving(args)
    print(f"serving: {ms_s * 1e3:.1f} us per prefill + {K_s} decode steps", file=sys.stderr,
          flush=True)
    small = {}
    for n in (1, 2):
        wn, hot, flushed, graph_ms, kern_n, P_n = bench_causal_small(args, n)
        small[n] = (wn, hot, flushed, graph_ms, kern_n, P_n)
        print(f"workload {n} ({wn.name}): hot {hot * 1e3:.1f} us, flushed {flushed * 1e3:.1f} us, "
              f"graph-replayed {graph_ms * 1e3:.1f} us; "
              "kernels " + ", ".join(f"{name} {t:.1f}" for name, t in
                                     kernels_us(kern_n, P_n, wn.dtype != "bf16").items())
              + " us", file=sys.stderr, flush=True)

    w, ms, ms_hot, wall, byts, flops, P, kern_ms, ms_steady = bench_prefill(args)
    print(f"prefill: {ms * 1e3:.1f} us/step (hot {ms_hot * 1e3:.1f} us); kernels "
          f"agg {kern_ms[0] * 1e3:.1f} causal {kern_ms[2] * 1e3:.1f} us",
          file=sys.stderr, flush=True)
    th = w.B * w.H * w.N
    value = th / (ms * 1e-3)
    achieved = byts / (kern_ms[2] * 1e-3)
    copy_bw = copy_bandwidth()
    d2d_bw = d2d_bandwidth()
    traffic = recorded_traffic()
    issued = mfma_issued_prefill(w.B, w.H, w.N, P)

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s (B*H*N/s)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "form": "causal", "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "d_v": w.dv, "chunk": args.chunk or 64, "segments_per_head": P,
                   "global_batch": w.B, "seq_len": w.N, "parallelism": "none (1 GPU)",
                   "input_sets_rotated": args.rotate},
        "roofline": {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK,
                     "traffic": traffic["bytes_per_launch"] if traffic else None,
                     "kernel": "k_causal<128, 0, false, false> (causal outputs + final state; reads q, k, v and "
                               "the segment sums before each segment, writes out and S, z)",
                     "kernel_us": kern_ms[2] * 1e3,
                     "algorithmic_bytes_per_launch": byts,
                     "copy_GBps": copy_bw / 1e9, "frac_of_copy": achieved / copy_bw,
                     "d2d_copy_GBps": d2d_bw / 1e9, "frac_of_d2d_copy": achieved / d2d_bw,
                     "call_us": ms * 1e3, "call_frac": byts / (ms * 1e-3) / HBM_PEAK,
                     "call_kernels_us": kernels_us(kern_ms, P, False)},
        "mfma": {"algorithmic_frac": flops / (ms * 1e-3) / BF16_PEAK,
                 "issued_frac": issued / (ms * 1e-3) / BF16_PEAK,
                 "peak_tflops": BF16_PEAK / 1e12},
        "hot_cache_ms_per_step": ms_hot,
        "steady_state": None if ms_steady is None else {
            "ms_per_step": ms_steady, "token_heads_per_s": th / (ms_steady * 1e-3),
            "warmup": args.steady, "steps": args.steady,
            "hbm_frac": byts / (ms_steady * 1e-3) / HBM_PEAK},
        "decode": {"workload": wd.name, "us_per_step": ms_d * 1e3,
                   "GB_per_s": byts_d / (ms_d * 1e-3) / 1e9,
                   "hbm_frac": byts_d / (ms_d * 1e-3) / HBM_PEAK,
                   "rmw_GBps": rmw_bw / 1e9, "frac_of_rmw": byts_d / (ms_d * 1e-3) / rmw_bw,
                   "steps": args.decode_steps},
        "global": {"workload": wg.name, "us_per_call": ms_g * 1e3,
                   "token_heads_per_s": wg.B * wg.H * wg.N / (ms_g * 1e-3),
                   "hbm_frac": byts_g / (ms_g * 1e-3) / HBM_PEAK,
                   "copy_GBps": copy_bw / 1e9, "frac_of_copy": byts_g / (ms_g * 1e-3) / copy_bw,
                   # the algorithmic flops of the two passes: 4 d d_v + 3 d + d_v per token-head
                   "mfma": {"algorithmic_frac": wg.B * wg.H * wg.N * (4 * wg.d * wg.dv + 3 * wg.d + wg.dv)
                            / (ms_g * 1e-3) / BF16_PEAK,
                            "busy_profile": "profiles/global_b1h8n100000_d128_mfma_busy.txt"}},
        "favor": {"workload": favor_name(), "m": m_f,
                  "us_per_step": ms_f * 1e3,
                  "token_heads_per_s": wf.B * wf.H * wf.N / (ms_f * 1e-3),
                  "algorithmic_hbm_frac": wf.B * wf.H * wf.N * (4 * wf.d * 2) / (ms_f * 1e-3) / HBM_PEAK,
                  "two_pass_us_per_step": ms_f2 * 1e3,
                  "features_us_per_tensor": ms_rf * 1e3,
                  "features_hbm_frac": rf_bytes / (ms_rf * 1e-3) / HBM_PEAK,
                  "two_pass_attention_kernels_us": kernels_us(kern_f, P, False)},
        "identity_unnormalized": {"workload": wv.name, "us_per_call": ms_v * 1e3,
                                  "token_heads_per_s": wv.B * wv.H * wv.N / (ms_v * 1e-3)},
        "float32": {"workload": w32.name.replace("_bf16", "_f32"), "entry_point": "la_causal_fwd_ws",
                    "chunk": 32, "segments_per_head": P_32, "us_per_call": ms_32 * 1e3,
                    "token_heads_per_s": w32.B * w32.H * w32.N / (ms_32 * 1e-3),
                    "kernels_us": kernels_us(kern_32, P_32, True),
                    # the float32 call is bound by the float32 matrix rate (its algorithmic
                    # bytes take 67 us at 8 TB/s, its issued products 177 us at 157.3 TFLOP/s)
                    "roofline": {"bound": "mfma", "unit": "TFLOP/s",
                                 "achieved": mfma32_issued_prefill(w32.B, w32.H, w32.N, P_32, w32.d)
                                 / (ms_32 * 1e-3) / 1e12,
                                 "peak": FP32_MFMA_PEAK / 1e12,
                                 "frac": mfma32_issued_prefill(w32.B, w32.H, w32.N, P_32, w32.d)
                                 / (ms_32 * 1e-3) / FP32_MFMA_PEAK,
                                 "scope": "whole call (segment sums, scan, causal), issued "
                                          "16x16x4 float32 products",
                                 "algorithmic_frac": algo_prefill(w32.B, w32.H, w32.N, w32.d, w32.dv, 4)[1]
                                 / (ms_32 * 1e-3) / FP32_MFMA_PEAK}},
        "retention": {"workload": retention_name(), "us_per_call": ms_r * 1e3,
                      "token_heads_per_s": wr.B * wr.H * wr.N / (ms_r * 1e-3)},
        "serving": {"workload": f"prefill {ws_.name} then {K_s} decode steps (HIP graph)",
                    "us_per_serving_step": ms_s * 1e3, "prefill_us": ms_sp * 1e3,
                    "decode_us_per_step": (ms_s - ms_sp) * 1e3 / K_s,
                    "token_heads_per_s": ws_.B * ws_.H * (ws_.N + K_s) / (ms_s * 1e-3)},
        "wall_s_timed_region": wall,
    }
    workloads = {}
    for n, (wn, hot, flushed, graph_ms, kern_n, P_n) in small.items():
        th_n = wn.B * wn.H * wn.N
        es = 2 if wn.dtype == "bf16" else 4
        byts_n = algo_prefill(wn.B, wn.H, wn.N, wn.d, wn.dv, es)[0]
        entry = {"form": "causal", "dtype": wn.dtype, "chunk": wn.chunk or None,
                 "segments_per_head": P_n, "entry_point": "la_causal_fwd_ws",
                 "us_per_call_hot": hot * 1e3, "us_per_call_flushed": flushed * 1e3,
                 # device time per call with the host's per-call cost taken out (replayed from a
                 # HIP graph of GRAPH_CALLS calls)
                 "us_per_call_graph": graph_ms * 1e3,
                 "token_heads_per_s_flushed": th_n / (flushed * 1e-3),
                 "kernels_us": kernels_us(kern_n, P_n, wn.dtype != "bf16"),
                 "algorithmic_bytes_per_call": byts_n,
                 "call_hbm_frac_flushed": byts_n / (flushed * 1e-3) / HBM_PEAK}
        if wn.dtype == "bf16":
            entry["roofline"] = {"bound": "hbm", "kernel": f"k_causal<{wn.d}, 0, false, false>",
                                 "achieved": byts_n / (kern_n[2] * 1e-3) / 1e9,
                                 "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                                 "frac": byts_n / (kern_n[2] * 1e-3) / HBM_PEAK,
                                 "note": "kernel timed hot (inputs fit in the last-level cache)"}
        else:
            entry["bound"] = "launch latency (64 token-heads, one launch)"
        workloads[wn.name] = entry
    workloads[wd.name] = rec.pop("decode")
    workloads[wg.name] = rec.pop("global")
    rec["workloads"] = workloads
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline()
        workloads[small[1][0].name]["cpu_baseline"] = cpu_baseline_causal(1, 2.0)
        workloads[small[2][0].name]["cpu_baseline"] = cpu_baseline_causal(2, 5.0)
        print("cpu baselines: workloads 1, 2 done", file=sys.stderr, flush=True)
        workloads[wg.name]["cpu_baseline"] = cpu_baseline_global()
        print("cpu baselines: global done", file=sys.stderr, flush=True)
        workloads[wd.name]["cpu_baseline"] = cpu_baseline_decode()
        print("cpu baselines: decode done", file=sys.stderr, flush=True)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
