"""GPU: the prefill -> decode hand-off (a serving loop) against the float64 oracle, and decode
steps captured in a HIP graph and replayed.

The state a prefill writes is the state the decode steps continue from, so the outputs of a
prefill over N tokens followed by K decode steps must equal the causal form over N + K tokens
("线性注意力从头到尾讲清楚", section 7: only S_t and z_t are kept between tokens; "Linear
Attention Math", section "The recurrent form": constant work per generated token).
"""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import DEV, check, f64, la, say, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


@pytest.mark.parametrize("dtype,d,N,K", [("bf16", 128, 1000, 40), ("bf16", 64, 2048, 24),
                                         ("f32", 32, 333, 20)])
def test_prefill_then_decode(dtype, d, N, K):
    B, H = 2, 4
    q, k, v = datagen.qkv(B, H, N + K, d, d, 1300 + d, 1 / math.sqrt(d), dtype)
    say(f"prefill {N} then {K} decode steps dtype={dtype} d={d}")
    mod = la()
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    out = torch.empty((B, H, N, d), dtype=q.dtype, device=DEV)
    S = torch.full((B, H, d, d), float("nan"), device=DEV)
    z = torch.full((B, H, d), float("nan"), device=DEV)
    mod.la_causal_fwd_state(qd[:, :, :N].contiguous(), kd[:, :, :N].contiguous(),
                            vd[:, :, :N].contiguous(), out, None, None, S, z)
    outs = torch.empty((K, B, H, d), dtype=q.dtype, device=DEV)
    for t in range(K):
        mod.la_decode_step(qd[:, :, N + t].contiguous(), kd[:, :, N + t].contiguous(),
                           vd[:, :, N + t].contiguous(), outs[t], S, z)
    torch.cuda.synchronize()
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v))
    check("prefill out", f64(out), oo[:, :, :N], TOL[dtype])
    check("decode outs", np.moveaxis(f64(outs), 0, 2), oo[:, :, N:], TOL[dtype])
    check("final S", f64(S), So, TOL[dtype])
    check("final z", f64(z), zo, TOL[dtype])


def test_decode_graph_replay():
    """K decode steps captured once in a HIP graph; every replay (from the same restored
    state, with eager work and synchronisation between replays) gives the eager results."""
    B, H, d, N, K = 4, 8, 128, 512, 16
    q, k, v = datagen.qkv(B, H, N, d, d, 1401, 1 / math.sqrt(d), "bf16")
    toks = [to_dev(x) for x in datagen.qkv(K, B * H, 1, d, d, 1402, 1 / math.sqrt(d), "bf16")]
    toks = [x.view(K, B, H, d) for x in toks]
    mod = la()
    say("decode graph: prefill, eager decode")
    out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=DEV)
    S = torch.empty((B, H, d, d), device=DEV)
    z = torch.empty((B, H, d), device=DEV)
    mod.la_causal_fwd_state(to_dev(q), to_dev(k), to_dev(v), out, None, None, S, z)
    S_pre, z_pre = S.clone(), z.clone()
    douts = torch.empty((K, B, H, d), dtype=torch.bfloat16, device=DEV)

    def decode_all():
        for t in range(K):
            mod.la_decode_step(toks[0][t], toks[1][t], toks[2][t], douts[t], S, z)

    decode_all()
    torch.cuda.synchronize()
    eager = douts.clone()
    S_end, z_end = S.clone(), z.clone()
    say("decode graph: capture")
    S.copy_(S_pre)
    z.copy_(z_pre)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode_all()
    torch.cuda.synchronize()
    for r in range(3):
        say(f"decode graph: replay {r}")
        S.copy_(S_pre)
        z.copy_(z_pre)
        douts.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(douts, eager), r
        assert torch.equal(S, S_end) and torch.equal(z, z_end), r
    # and the eager outputs themselves are right
    qq, kk, vv = (torch.cat([a, b.permute(1, 2, 0, 3).reshape(B, H, K, d).cpu()], dim=2)
                  for a, b in zip((q, k, v), toks))
    oo, _, _, _, _ = oracle.causal(f64(qq), f64(kk), f64(vv))
    check("decode outs", np.moveaxis(f64(eager), 0, 2), oo[:, :, N:], TOL["bf16"])
