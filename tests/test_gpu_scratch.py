"""GPU tests of the library's scratch memory: segment states live in blocks cached per
(device, stream), so calls must stay correct when a stream's shapes grow and shrink, when
calls on two streams interleave without synchronisation, and when a call is captured into a
graph (its scratch then comes from a stream-ordered pool)."""
from __future__ import annotations

import math

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
