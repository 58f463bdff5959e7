"""GPU tests of the library's scratch memory: segment states live in blocks cached per
(device, stream), so calls must stay correct when a stream's shapes grow and shrink, when
calls on two streams interleave without synchronisation, and when a call is captured into a
graph (its scratch then comes from a stream-ordered pool)."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import DEV, check, f64, la, say, to_dev

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-5}


def _inputs(B, H, N, d, seed, dtype="bf16"):
    return datagen.qkv(B, H, N, d, d, seed, 1 / math.sqrt(d), dtype)


def _run(mod, q, k, v, seg_len, S0=None, z0=None):
    """One causal call on the current stream into fresh device buffers (no synchronisation)."""
    B, H, N, d = q.shape
    out = torch.empty((B, H, N, d), dtype=q.dtype, device=DEV)
    S = torch.full((B, H, d, d), float("nan"), device=DEV)
    z = torch.full((B, H, d), float("nan"), device=DEV)
    mod.la_causal_fwd_state(q, k, v, out, S0, z0, S, z, seg_len=seg_len)
    return out, S, z


def _check_oracle(name, q, k, v, out, S, z, dtype="bf16"):
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v))
    check(f"{name} out", f64(out), oo, TOL[dtype])
    check(f"{name} S", f64(S), So, TOL[dtype])
    check(f"{name} z", f64(z)[..., None], zo[..., None], TOL[dtype])


def test_scratch_shapes_grow_and_shrink():
    """One stream, workspace needs of 1x, 6x, 1x, 12x, 3x the first call's (segments of 128
    tokens): every result matches the oracle."""
    mod = la()
    for i, (H, N) in enumerate([(1, 512), (3, 1024), (1, 512), (3, 2048), (3, 512)]):
        q, k, v = _inputs(1, H, N, 64, 300 + i)
        say(f"scratch grow/shrink call {i}: H={H} N={N} d=64 seg_len=128")
        out, S, z = _run(mod, to_dev(q), to_dev(k), to_dev(v), 128)
        torch.cuda.synchronize()
        _check_oracle(f"call {i}", q, k, v, out, S, z)


def test_scratch_two_streams_interleaved():
    """Calls alternate between two streams with no synchronisation in between; each stream
    keeps its own scratch, so every result matches the oracle."""
    mod = la()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    cases = []
    for i in range(6):
        q, k, v = _inputs(2, 2, 1536 + 256 * (i % 3), 128, 400 + i)
        cases.append((q, k, v, to_dev(q), to_dev(k), to_dev(v)))
    torch.cuda.synchronize()
    res = []
    say("scratch two streams: 6 calls alternating, d=128, seg_len=256")
    for i, (_, _, _, qd, kd, vd) in enumerate(cases):
        s = streams[i % 2]
        with torch.cuda.stream(s):
            res.append(_run(mod, qd, kd, vd, 256))
    torch.cuda.synchronize()
    for i, ((q, k, v, _, _, _), (out, S, z)) in enumerate(zip(cases, res)):
        _check_oracle(f"stream {i % 2} call {i}", q, k, v, out, S, z)


def test_scratch_under_graph_capture():
    """A causal call captured into a graph (scratch from the stream-ordered pool) replays to
    the eager result, bit for bit, with eager calls (cached scratch) between the replays."""
    mod = la()
    q, k, v = _inputs(2, 4, 3000, 128, 500)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    say("scratch graph capture: causal call B=2 H=4 N=3000 d=128 seg_len=512")
    out_e, S_e, z_e = _run(mod, qd, kd, vd, 512)
    torch.cuda.synchronize()
    _check_oracle("eager", q, k, v, out_e, S_e, z_e)
    out_g = torch.empty_like(out_e)
    S_g = torch.empty_like(S_e)
    z_g = torch.empty_like(z_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mod.la_causal_fwd_state(qd, kd, vd, out_g, None, None, S_g, z_g, seg_len=512)
    q2, k2, v2 = (to_dev(x) for x in _inputs(2, 4, 3000, 128, 501))
    for rep in range(3):
        out_g.zero_()
        S_g.zero_()
        z_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        say(f"  replay {rep}")
        assert torch.equal(out_g, out_e), f"replay {rep}: out differs from the eager call"
        assert torch.equal(S_g, S_e) and torch.equal(z_g, z_e), f"replay {rep}: state differs"
        # eager work on the same device between replays, through the cached scratch
        _run(mod, q2, k2, v2, 512)
        torch.cuda.synchronize()



@pytest.mark.parametrize("decay", [False, True])
def test_graph_capture_initial_state_in_place(decay):
    """A causal call with the initial state passed in S, z (read, then overwritten with the
    final state; several segments, so the segment-sum kernel first copies the initial state
    into the scratch for the causal kernel) captured into a graph. S, z are restored before
    each replay, with eager calls between the replays: every replay equals the eager call bit
    for bit, and the eager call matches the oracle."""
    mod = la()
    B, H, N, d, n0 = 2, 4, 3000, 128, 64
    q, k, v = _inputs(B, H, N + n0, d, 520 + decay)
    gamma = np.linspace(0.95, 1.0, H) if decay else None
    _, S0, z0, _, _ = oracle.causal(f64(q[:, :, :n0]), f64(k[:, :, :n0]), f64(v[:, :, :n0]),
                                    gamma=gamma)
    S0d = torch.from_numpy(S0.astype(np.float32)).to(DEV)
    z0d = torch.from_numpy(z0.astype(np.float32)).to(DEV)
    q, k, v = (x[:, :, n0:].contiguous() for x in (q, k, v))
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    g_dev = None if gamma is None else torch.from_numpy(gamma.astype(np.float32)).to(DEV)

    def call(out, S, z):
        if decay:
            mod.la_causal_fwd_decay(qd, kd, vd, out, g_dev, S, z, S, z, seg_len=512)
        else:
            mod.la_causal_fwd(qd, kd, vd, out, S, z, seg_len=512)

    say(f"graph capture, initial state in place: B={B} H={H} N={N} d={d} seg_len=512 decay={decay}")
    out_e = torch.empty_like(qd)
    S_e, z_e = S0d.clone(), z0d.clone()
    call(out_e, S_e, z_e)
    torch.cuda.synchronize()
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v), S0=S0.astype(np.float32),
                                     z0=z0.astype(np.float32), gamma=gamma)
    check("eager out", f64(out_e), oo, TOL["bf16"])
    check("eager S", f64(S_e), So, TOL["bf16"])
    out_g = torch.empty_like(qd)
    S_g, z_g = S0d.clone(), z0d.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out_g, S_g, z_g)
    q2, k2, v2 = (to_dev(x) for x in _inputs(B, H, N, d, 530))
    for rep in range(3):
        S_g.copy_(S0d)
        z_g.copy_(z0d)
        out_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        say(f"  replay {rep}")
        assert torch.equal(out_g, out_e), f"replay {rep}: out differs from the eager call"
        assert torch.equal(S_g, S_e) and torch.equal(z_g, z_e), f"replay {rep}: state differs"
        _run(mod, q2, k2, v2, 512, S0d, z0d)
        torch.cuda.synchronize()


def test_scratch_host_threads():
    """Four host threads, each with its own stream, enqueue causal calls at the same time (the
    binding releases the interpreter lock during the C call); every result matches the oracle."""
    import threading
    mod = la()
    cases = [_inputs(1, 2, 1024 + 128 * i, 64, 700 + i) for i in range(4)]
    dev_in = [tuple(to_dev(x) for x in c) for c in cases]
    torch.cuda.synchronize()
    results = [None] * 4
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = [_run(mod, *dev_in[i], 128) for _ in range(3)]
            s.synchronize()
            results[i] = outs
        except Exception as e:  # reported below, on the main thread
            errors.append(e)

    say("scratch host threads: 4 threads x 3 calls, d=64, seg_len=128")
    threads = [threading.Thread(target=work, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, (q, k, v) in enumerate(cases):
        for j, (out, S, z) in enumerate(results[i]):
            _check_oracle(f"thread {i} call {j}", q, k, v, out, S, z)


# ---------------------------------------------------------------- caller-supplied workspace
def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("dtype,d,seg,decay", [("bf16", 128, 0, False), ("bf16", 64, 128, False),
                                               ("f32", 32, 64, False), ("bf16", 128, 256, True),
                                               ("f32", 128, 0, False), ("f32", 64, 96, True)])
def test_workspace_causal(dtype, d, seg, decay):
    """la_causal_fwd_ws with the segment states in a caller-owned buffer that starts as NaN
    (no part of it needs an initial value): the oracle's results, and bit-identical to the
    convenience form with the library's scratch."""
    mod = la()
    B, H, N = 2, 3, 1500
    q, k, v = _inputs(B, H, N, d, 810 + d, dtype)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    gam = torch.tensor([0.9, 0.99, 0.5], dtype=torch.float32, device=DEV) if decay else None
    need = mod.la_workspace_bytes(0, B, H, N, d, d, 0, seg, datagen_code(dtype))
    assert need > 0
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=DEV)
    say(f"workspace causal dtype={dtype} d={d} seg={seg} decay={decay} ws={need} B")
    res = []
    for use_ws in (True, False):
        out = torch.full((B, H, N, d), float("nan"), dtype=q.dtype, device=DEV)
        S = torch.full((B, H, d, d), float("nan"), device=DEV)
        z = torch.full((B, H, d), float("nan"), device=DEV)
        if use_ws:
            mod.la_causal_fwd_ws(qd, kd, vd, out, ws, None, None, S, z, gamma=gam, seg_len=seg)
        elif decay:
            mod.la_causal_fwd_decay(qd, kd, vd, out, gam, None, None, S, z, seg_len=seg)
        else:
            mod.la_causal_fwd_ex(qd, kd, vd, out, None, None, S, z, seg_len=seg)
        torch.cuda.synchronize()
        res.append((out, S, z))
    for a, b in zip(*res):
        assert torch.equal(_bits(a), _bits(b)), "workspace form differs from the cached form"
    gnp = None if gam is None else gam.cpu().numpy().astype(np.float64)
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v), gamma=gnp)
    out, S, z = res[0]
    check("out", f64(out), oo, TOL[dtype])
    check("S", f64(S), So, TOL[dtype])
    check("z", f64(z)[..., None], zo[..., None], TOL[dtype])


@pytest.mark.parametrize("dtype,d,N", [("bf16", 128, 20000), ("f32", 64, 3000)])
def test_workspace_global(dtype, d, N):
    mod = la()
    B, H = 1, 2
    q, k, v = _inputs(B, H, N, d, 830 + d, dtype)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    need = mod.la_workspace_bytes(1, B, H, N, d, d, 0, 0, datagen_code(dtype))
    assert need > 0
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=DEV)
    say(f"workspace global dtype={dtype} d={d} N={N} ws={need} B")
    res = []
    for use_ws in (True, False):
        out = torch.full((B, H, N, d), float("nan"), dtype=q.dtype, device=DEV)
        S = torch.full((B, H, d, d), float("nan"), device=DEV)
        z = torch.full((B, H, d), float("nan"), device=DEV)
        if use_ws:
            mod.la_global_fwd_ws(qd, kd, vd, out, S, z, ws)
        else:
            mod.la_global_fwd(qd, kd, vd, out, S, z)
        torch.cuda.synchronize()
        res.append((out, S, z))
    for a, b in zip(*res):
        assert torch.equal(_bits(a), _bits(b)), "workspace form differs from the cached form"
    oo, So, zo, _, _ = oracle.global_(f64(q), f64(k), f64(v))
    out, S, z = res[0]
    check("out", f64(out), oo, TOL[dtype])
    check("S", f64(S), So, TOL[dtype])


def test_workspace_graph_capture():
    """A la_causal_fwd_ws call captured into a HIP graph (kernel nodes only) and replayed, with
    eager calls between the replays: every replay equals the eager result bit for bit."""
    mod = la()
    q, k, v = _inputs(1, 4, 2048, 128, 850)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    need = mod.la_workspace_bytes(0, 1, 4, 2048, 128, 128, 0, 256, 1)
    ws = torch.empty(need // 4, dtype=torch.float32, device=DEV)
    out_e = torch.empty_like(qd)
    S_e = torch.empty(1, 4, 128, 128, device=DEV)
    z_e = torch.empty(1, 4, 128, device=DEV)
    say("workspace graph capture")
    mod.la_causal_fwd_ws(qd, kd, vd, out_e, ws, None, None, S_e, z_e, seg_len=256)
    torch.cuda.synchronize()
    out_g = torch.empty_like(qd)
    S_g = torch.empty_like(S_e)
    z_g = torch.empty_like(z_e)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mod.la_causal_fwd_ws(qd, kd, vd, out_g, ws, None, None, S_g, z_g, seg_len=256)
    torch.cuda.synchronize()
    q2, k2, v2 = (to_dev(x) for x in _inputs(1, 4, 2048, 128, 851))
    for rep in range(3):
        out_g.fill_(float("nan"))
        S_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out_g), _bits(out_e)), f"replay {rep}: outputs differ"
        assert torch.equal(S_g, S_e) and torch.equal(z_g, z_e), f"replay {rep}: state differs"
        # eager work through the same workspace between replays
        o2 = torch.empty_like(q2)
        mod.la_causal_fwd_ws(q2, k2, v2, o2, ws, seg_len=256)
        torch.cuda.synchronize()


def test_per_thread_streams():
    """Two host threads, both on the per-thread default stream (one handle, a different stream
    in each thread), each enqueue calls of changing sizes without synchronising: scratch is
    reused only after its last use has finished, so every result equals the single-stream
    result bit for bit."""
    import ctypes
    import threading
    mod = la()
    per_thread = ctypes.c_void_p(2)  # hipStreamPerThread
    shapes = [(1, 2, 1024 + 256 * i, 64) for i in range(4)]
    cases = [tuple(to_dev(x) for x in _inputs(*sh, 870 + i)) for i, sh in enumerate(shapes)]
    want = []
    for q, k, v in cases:
        want.append(_run(mod, q, k, v, 128))
    torch.cuda.synchronize()
    results = {}
    errors = []

    def work(tid):
        try:
            for rep in range(6):
                i = (rep + tid) % len(cases)
                q, k, v = cases[i]
                B, H, N, d = q.shape
                out = torch.full((B, H, N, d), float("nan"), dtype=q.dtype, device=DEV)
                S = torch.full((B, H, d, d), float("nan"), device=DEV)
                z = torch.full((B, H, d), float("nan"), device=DEV)
                st = mod.lib.la_causal_fwd_state(
                    q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), None, None,
                    S.data_ptr(), z.data_ptr(), B, H, N, d, d, 0, 128, mod.LA_BF16, per_thread)
                assert st == mod.LA_OK, st
                results[(tid, rep)] = (i, out, S, z)
        except Exception as e:  # reported below, on the main thread
            errors.append(e)

    torch.cuda.synchronize()
    say("per-thread streams: 2 threads x 6 calls, d=64, seg_len=128")
    threads = [threading.Thread(target=work, args=(t,)) for t in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for (tid, rep), (i, out, S, z) in results.items():
        wo, wS, wz = want[i]
        assert torch.equal(_bits(out), _bits(wo)), (tid, rep)
        assert torch.equal(S, wS) and torch.equal(z, wz), (tid, rep)


def test_release_cache():
    """la_release_cache frees the cached blocks; later calls allocate anew and stay correct."""
    mod = la()
    q, k, v = (to_dev(x) for x in _inputs(1, 4, 3000, 128, 880))
    say("release cache")
    a = _run(mod, q, k, v, 512)
    mod.la_release_cache()
    b = _run(mod, q, k, v, 512)
    mod.la_release_cache()
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(_bits(x), _bits(y))


def datagen_code(dtype):
    return 1 if dtype == "bf16" else 0
