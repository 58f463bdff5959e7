"""GPU parity of the float32 matrix-core kernels (d = d_v in {64, 128}, chunks of 32 tokens)
against the float64 oracle at the float32 tolerance: ragged lengths around the chunk size,
segment splits, a state carried between calls, the global form, the headline shape in float32,
and repeatability. (Flags with a carried state are covered by tests/test_gpu_variants.py, the
decayed float32 call, which runs the vector-ALU kernels on the same plan, by
tests/test_gpu_decay.py.)"""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import causal, check, f64, global_, say, to_dev, DEV, la

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.mark.parametrize("d,N", [(128, 1), (128, 31), (128, 33), (128, 1000), (64, 1), (64, 95),
                                 (64, 2000)])
def test_f32_causal_and_global_ragged(d, N):
    q, k, v = datagen.qkv(2, 3, N, d, d, 900 + N + d, 1 / math.sqrt(d), "f32")
    say(f"f32 matrix ragged d={d} N={N}")
    o, S, z = causal(q, k, v)
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v))
    check("out", o, oo, TOL)
    check("S", S, So, TOL)
    check("z", z, zo, TOL)
    og, Sg, zg = global_(q, k, v)
    oo, So, zo, _, _ = oracle.global_(f64(q), f64(k), f64(v))
    check("global out", og, oo, TOL)
    check("global S", Sg, So, TOL)
    check("global z", zg, zo, TOL)


@pytest.mark.parametrize("seg", [32, 96, 512, 0])
def test_f32_segment_split(seg):
    """Any split of the sequence into segments gives the same result (to rounding)."""
    q, k, v = datagen.qkv(1, 4, 4096 + 40, 128, 128, 17, 1 / math.sqrt(128), "f32")
    say(f"f32 matrix segment split seg_len={seg}")
    o, S, z = causal(q, k, v, seg_len=seg)
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v))
    check("out", o, oo, TOL)
    check("S", S, So, TOL)


@pytest.mark.parametrize("d", [64, 128])
def test_f32_state_carry(d):
    """Two calls with the state carried through S, z equal one call over the whole sequence."""
    N, n1 = 700, 333
    q, k, v = datagen.qkv(2, 2, N, d, d, 23 + d, 1 / math.sqrt(d), "f32")
    qa, ka, va = (x[:, :, :n1].contiguous() for x in (q, k, v))
    qb, kb, vb = (x[:, :, n1:].contiguous() for x in (q, k, v))
    say(f"f32 matrix state carry d={d}")
    oa, Sa, za = causal(qa, ka, va)
    ob, Sb, zb = causal(qb, kb, vb, S0=Sa.astype(np.float32), z0=za.astype(np.float32))
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v))
    check("two-piece out", np.concatenate([oa, ob], axis=2), oo, TOL)
    check("two-piece S", Sb, So, TOL)
    check("two-piece z", zb, zo, TOL)


def test_f32_headline_shape():
    """B=2 H=16 N=8192 d=128 in float32: every output row, S and z."""
    q, k, v = datagen.qkv(2, 16, 8192, 128, 128, 1003, 1 / math.sqrt(128), "f32")
    say("f32 matrix B=2 H=16 N=8192 d=128")
    o, S, z = causal(q, k, v)
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v))
    check("out", o, oo, TOL)
    check("S", S, So, TOL)
    check("z", z, zo, TOL)


def test_f32_repeatable():
    """Two identical calls give bit-identical outputs and states (fixed reduction order)."""
    q, k, v = datagen.qkv(1, 8, 3000, 128, 128, 31, 1 / math.sqrt(128), "f32")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    say("f32 matrix repeatable")
    res = []
    for _ in range(2):
        out = torch.empty_like(qd)
        # S, z carry the initial state in and the final state out
        S = torch.zeros((1, 8, 128, 128), dtype=torch.float32, device=DEV)
        z = torch.zeros((1, 8, 128), dtype=torch.float32, device=DEV)
        la().la_causal_fwd(qd, kd, vd, out, S, z)
        og = torch.empty_like(qd)
        Sg = torch.empty_like(S)
        zg = torch.empty_like(z)
        la().la_global_fwd(qd, kd, vd, og, Sg, zg)
        torch.cuda.synchronize()
        res.append((out, S, z, og, Sg, zg))
    for a, b in zip(*res):
        assert torch.equal(a, b)
