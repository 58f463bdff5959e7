"""GPU parity of the variant forms against the float64 oracle: identity feature map and the
unnormalised read (the *_ex entry points), positive random features (la_rf_features), and
attention over random features.

Criteria: row-wise max-norm relative error (oracle/compare.py) within 1e-5 for float32 and
2e-2 for bfloat16, as for the base forms; the feature map element by element within its
rounding bound (one bf16 rounding plus float32 argument error for bf16; 2e-5 for float32).
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
EXACT_TOL = {"f32": 2e-7, "bf16": 2.0 ** -8}
IDENT, UNNORM = 1, 2
MODE = {0: ("elu1", True), IDENT: ("identity", True), UNNORM: ("elu1", False),
        IDENT | UNNORM: ("identity", False)}

# (dtype, d, chunk): matrix-core (bf16, d in {64, 128}, chunk 64) and vector-ALU kernels
PATHS = [("bf16", 128, 0), ("bf16", 64, 0), ("f32", 32, 16), ("bf16", 16, 32), ("f32", 128, 32),
         ("f32", 64, 0), ("f32", 128, 16)]


def causal_ex(q, k, v, flags, S0=None, z0=None, chunk=0, seg_len=0):
    B, H, N, d = q.shape
    dv = v.shape[-1]
    out = torch.empty((B, H, N, dv), dtype=q.dtype, device=DEV)
    S = torch.full((B, H, d, dv), float("nan"), device=DEV)
    z = torch.full((B, H, d), float("nan"), device=DEV)
    S0d = None if S0 is None else torch.as_tensor(S0, dtype=torch.float32).to(DEV)
    z0d = None if z0 is None else torch.as_tensor(z0, dtype=torch.float32).to(DEV)
    la().la_causal_fwd_ex(to_dev(q), to_dev(k), to_dev(v), out, S0d, z0d, S, z, chunk=chunk,
                          seg_len=seg_len, flags=flags)
    torch.cuda.synchronize()
    return f64(out), f64(S), f64(z)


def global_ex(q, k, v, flags, chunk=0):
    B, H, N, d = k.shape
    dv = v.shape[-1]
    out = torch.empty((B, H, q.shape[2], dv), dtype=k.dtype, device=DEV)
    S = torch.full((B, H, d, dv), float("nan"), device=DEV)
    z = torch.full((B, H, d), float("nan"), device=DEV)
    la().la_global_fwd_ex(to_dev(q), to_dev(k), to_dev(v), out, S, z, chunk=chunk, flags=flags)
    torch.cuda.synchronize()
    return f64(out), f64(S), f64(z)


def _inputs(flags, B, H, N, d, dv, seed, dtype):
    """ELU+1 forms take N(0, 1/d) inputs; identity forms with a division take strictly
    positive features (so every denominator is a sum of positive terms); identity without a
    division takes signed values."""
    if flags == IDENT:
        q = datagen.positive((B, H, N, d), seed, 1 / math.sqrt(d), dtype)
        k = datagen.positive((B, H, N, d), seed + 1, 1 / math.sqrt(d), dtype)
        v = datagen.normal((B, H, N, dv), seed + 2, 1.0, dtype)
        return q, k, v
    return datagen.qkv(B, H, N, d, dv, seed, 1 / math.sqrt(d), dtype)


# ---------------------------------------------------------------- worked examples natively
def _feat(rows, d, dtype):
    """Feature rows embedded in d columns (padding features 0), as [1, 1, N, d]."""
    rows = np.asarray(rows, dtype=np.float64)
    out = np.zeros((1, 1, rows.shape[0], d))
    out[0, 0, :, : rows.shape[1]] = rows
    return torch.from_numpy(out).to(datagen.DTYPES[dtype])


@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 128, 0), ("bf16", 64, 0), ("f32", 16, 16),
                                           ("bf16", 16, 32)])
def test_worked_examples_feature_space(golden, dtype, d, chunk):
    """The pages' examples are written in feature space; with the identity map they run as
    printed: the reads of S3 with and without the division, 10/3, and the global example."""
    g = golden("w7_unnormalised_reads.json")["state_example"]
    k = _feat(g["k"], d, dtype)
    v = _feat(g["v"], d, dtype)
    for qs, key in (([1, 0], "q=[1,0]"), ([0, 1], "q=[0,1]"), ([1, 1], "q=[1,1]")):
        q = _feat(np.vstack([g["k"][0], g["k"][1], qs]), d, dtype)
        say(f"S3 read {key} dtype={dtype} d={d} chunk={chunk}")
        o, S, z = causal_ex(q, k, v, IDENT | UNNORM, chunk=chunk)
        want = np.zeros((1, 1, 1, d))
        want[0, 0, 0, :2] = g["printed_reads"][key]
        check(f"unnormalised read {key}", o[:, :, 2:], want, EXACT_TOL[dtype])
        Sw = np.zeros((1, 1, d, d))
        Sw[0, 0, :2, :2] = golden("w2_three_token.json")["printed"]["S3"]
        check("S3", S, Sw, 1e-6)
    g2 = golden("w2_three_token.json")
    o, _, _ = causal_ex(k, k, v, IDENT, chunk=chunk)
    want = np.zeros((1, 1, 3, d))
    want[0, 0, :, :2] = g2["derived"]["causal_outputs_with_q_equal_k"]
    check("normalised causal outputs", o, want, EXACT_TOL[dtype])
    g1 = golden("w1_two_token_read.json")
    q1 = g1["q_at_position_1"]
    o, _, _ = causal_ex(_feat([q1, q1], d, dtype), _feat(g1["k"], d, dtype),
                        _feat(g1["v"], d, dtype), IDENT, chunk=chunk)
    want = np.zeros((1, 1, 2, d))
    want[0, 0, :, 0] = [g1["derived"]["output_at_position_0"], 10.0 / 3.0]
    check("10/3", o, want, EXACT_TOL[dtype])
    g6 = golden("w6_global_example.json")
    o, S, _ = global_ex(_feat(g6["q"], d, dtype), _feat(g6["k"], d, dtype), _feat(g6["v"], d, dtype),
                        IDENT, chunk=chunk)
    want = np.zeros((1, 1, 3, d))
    want[0, 0, :, :2] = g6["derived"]["global_outputs"]
    check("global example", o, want, EXACT_TOL[dtype])


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 16)])
def test_worked_example_decode_feature_space(golden, dtype, d):
    """The decode example with the identity map: numerator [3, 2] unnormalised, [0.75, 0.5]
    normalised, S and z as printed."""
    g = golden("w3_decode_example.json")
    for flags, want_vals in ((IDENT | UNNORM, g["printed"]["numerator"]), (IDENT, g["printed"]["output"])):
        S = torch.zeros((1, 1, d, d), dtype=torch.float32, device=DEV)
        z = torch.zeros((1, 1, d), dtype=torch.float32, device=DEV)
        q = to_dev(_feat([g["phi_q"]], d, dtype)[:, :, 0])
        for t in range(2):
            k = to_dev(_feat([g["phi_k"][t]], d, dtype)[:, :, 0])
            v = to_dev(_feat([g["v"][t]], d, dtype)[:, :, 0])
            out = torch.empty((1, 1, d), dtype=k.dtype, device=DEV)
            say(f"W3 decode flags={flags} step {t} dtype={dtype} d={d}")
            la().la_decode_step_ex(q, k, v, out, S, z, flags=flags)
        torch.cuda.synchronize()
        want = np.zeros((1, 1, d))
        want[0, 0, :2] = want_vals
        check("W3 out", f64(out), want, EXACT_TOL[dtype])
        Sw = np.zeros((1, 1, d, d))
        Sw[0, 0, :2, :2] = g["printed"]["S"]
        check("W3 S", f64(S), Sw, 1e-7)
        zw = np.zeros((1, 1, d))
        zw[0, 0, :2] = g["printed"]["z"]
        check("W3 z", f64(z)[..., None], zw[..., None], 1e-7)


# ---------------------------------------------------------------- random inputs, every flag
@pytest.mark.parametrize("flags", [IDENT, UNNORM, IDENT | UNNORM])
@pytest.mark.parametrize("dtype,d,chunk", PATHS)
def test_flags_causal_and_global(flags, dtype, d, chunk):
    """Several chunks and segments with a ragged tail, from a carried initial state."""
    B, H, N = 2, 3, 1000 + d
    q, k, v = _inputs(flags, B, H, N, d, d, 300 + d + flags, dtype)
    mode, norm = MODE[flags]
    n1 = 389
    say(f"flags={flags} dtype={dtype} d={d} chunk={chunk} N={N}")
    _, S1, z1, _, _ = oracle.causal(f64(q[:, :, :n1]), f64(k[:, :, :n1]), f64(v[:, :, :n1]),
                                    mode=mode, normalize=norm)
    S1, z1 = S1.astype(np.float32), z1.astype(np.float32)
    qb, kb, vb = (x[:, :, n1:].contiguous() for x in (q, k, v))
    o, S, z = causal_ex(qb, kb, vb, flags, S0=S1, z0=z1, chunk=chunk, seg_len=0)
    oo, So, zo, _, _ = oracle.causal(f64(qb), f64(kb), f64(vb), S0=S1, z0=z1, mode=mode,
                                     normalize=norm)
    check("causal out", o, oo, TOL[dtype])
    check("causal S", S, So, TOL[dtype])
    check("causal z", z, zo, TOL[dtype])   # rows = heads (signed features sum near 0)
    og, Sg, zg = global_ex(q, k, v, flags, chunk=chunk)
    oo, So, zo, _, _ = oracle.global_(f64(q), f64(k), f64(v), mode=mode, normalize=norm)
    check("global out", og, oo, TOL[dtype])
    check("global S", Sg, So, TOL[dtype])
    check("global z", zg, zo, TOL[dtype])


@pytest.mark.parametrize("flags", [IDENT, UNNORM, IDENT | UNNORM])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 32)])
def test_flags_decode(flags, dtype, d):
    B, H, steps = 4, 5, 3
    mode, norm = MODE[flags]
    q, k, v = _inputs(flags, B, H, steps + 40, d, d, 500 + d + flags, dtype)
    _, S0, z0, _, _ = oracle.global_(None, f64(k[:, :, :40]), f64(v[:, :, :40]), mode=mode)
    S0, z0 = S0.astype(np.float32), z0.astype(np.float32)
    S, z = torch.from_numpy(S0).to(DEV), torch.from_numpy(z0).to(DEV)
    So, zo = S0.astype(np.float64), z0.astype(np.float64)
    for t in range(40, 40 + steps):
        qt, kt, vt = (x[:, :, t].contiguous() for x in (q, k, v))
        out = torch.empty((B, H, d), dtype=qt.dtype, device=DEV)
        say(f"decode flags={flags} dtype={dtype} d={d} step {t}")
        la().la_decode_step_ex(to_dev(qt), to_dev(kt), to_dev(vt), out, S, z, flags=flags)
        torch.cuda.synchronize()
        oo, So, zo = oracle.decode_step(f64(qt), f64(kt), f64(vt), So, zo, mode=mode, normalize=norm)
        check(f"out step {t}", f64(out), oo, TOL[dtype])
    check("S", f64(S), So, 1e-6)
    check("z", f64(z), zo, 1e-6)   # rows = heads


def test_flags_zero_is_base_form():
    """flags = 0 gives exactly the base entry points' bytes."""
    q, k, v = datagen.qkv(2, 4, 2000, 128, 128, 61, 1 / math.sqrt(128), "bf16")
    say("flags 0 equals base form")
    a = causal_ex(q, k, v, 0)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    out = torch.empty_like(qd)
    S = torch.zeros((2, 4, 128, 128), device=DEV)
    z = torch.zeros((2, 4, 128), device=DEV)
    la().la_causal_fwd(qd, kd, vd, out, S, z)
    torch.cuda.synchronize()
    assert np.array_equal(a[0], f64(out))
    assert np.array_equal(a[1], f64(S))


# ---------------------------------------------------------------- positive random features
def rf_gpu(x, W):
    xd, Wd = to_dev(x), to_dev(W)
    f = torch.empty(tuple(x.shape[:-1]) + (W.shape[0],), dtype=x.dtype, device=DEV)
    la().la_rf_features(xd, Wd, f)
    torch.cuda.synchronize()
    return f


def check_rf(got, want, dtype):
    """Element-wise relative error of the features: one bf16 rounding (2^-9) plus a float32
    argument error for bf16; 2e-5 for float32."""
    tol = 2.0 ** -8 if dtype == "bf16" else 2e-5
    rel = np.abs(got - want) / np.abs(want)
    say(f"  features: max rel {rel.max():.3e} tol {tol:g} min {want.min():.3e} max {want.max():.3e}")
    assert np.all(np.isfinite(got)) and np.all(got > 0)
    assert rel.max() <= tol


@pytest.mark.parametrize("dtype,d,m,rows", [
    ("bf16", 128, 128, 1000), ("bf16", 128, 256, 129), ("bf16", 128, 64, 64), ("bf16", 64, 128, 1),
    ("bf16", 64, 64, 333), ("bf16", 64, 256, 70), ("bf16", 16, 16, 100), ("bf16", 128, 96, 65),
    ("f32", 32, 48, 100), ("f32", 128, 128, 77), ("f32", 7, 5, 33),
    # enough rows for the full grid (two 4-wave workgroups per CU at m = 128, one 8-wave
    # workgroup per CU at m = 256) with several 16-row tiles per wave and a ragged last tile
    ("bf16", 128, 128, 40003), ("bf16", 128, 256, 40003),
    # one partial tile for the 8-wave workgroup: seven of its waves find no tile to sweep
    ("bf16", 128, 256, 1), ("bf16", 128, 256, 15)])
def test_rf_features(dtype, d, m, rows):
    x = datagen.normal((rows, d), 700 + d + m, 1 / math.sqrt(d) * 1.5, dtype)
    W = datagen.projections(m, d, 800 + m, dtype)
    say(f"random features dtype={dtype} d={d} m={m} rows={rows}")
    f = f64(rf_gpu(x, W))
    check_rf(f, oracle.rf_map(f64(x), f64(W)), dtype)


def test_rf_features_large_norms():
    """Rows with |x|^2 up to ~40 (tiny features, no underflow to zero in float32 range)."""
    x = datagen.normal((512, 128), 901, 0.55, "bf16")
    W = datagen.projections(128, 128, 902, "bf16")
    say("random features, large norms")
    f = f64(rf_gpu(x, W))
    check_rf(f, oracle.rf_map(f64(x), f64(W)), "bf16")


def _favor(B, H, N, d, m, seed_qkv, seed_w, flags=IDENT):
    q, k, v = datagen.qkv(B, H, N, d, d, seed_qkv, 1 / math.sqrt(d), "bf16")
    W = datagen.projections(m, d, seed_w, "bf16")
    fq, fk = rf_gpu(q, W), rf_gpu(k, W)
    out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=DEV)
    S = torch.zeros((B, H, m, d), device=DEV)
    z = torch.zeros((B, H, m), device=DEV)
    la().la_causal_fwd_ex(fq, fk, to_dev(v), out, None, None, S, z, flags=flags)
    torch.cuda.synchronize()
    return (q, k, v, W), (f64(fq), f64(fk)), (f64(out), f64(S), f64(z))


@pytest.mark.parametrize("d,m,N", [(128, 128, 3000), (64, 64, 1111), (64, 128, 700)])
def test_favor_causal(d, m, N):
    """Random features of q and k, then causal identity-map attention over them, against the
    oracle's features and recurrence (m == d runs on the matrix cores; m != d on the
    vector-ALU kernel)."""
    say(f"favor causal d={d} m={m} N={N}")
    (q, k, v, W), _, (o, S, z) = _favor(2, 2, N, d, m, 1100 + d, 1200 + m)
    fq, fk = oracle.rf_map(f64(q), f64(W)), oracle.rf_map(f64(k), f64(W))
    oo, So, zo, _, _ = oracle.causal(fq, fk, f64(v), mode="identity")
    check("out", o, oo, TOL["bf16"])
    check("S", S, So, TOL["bf16"])
    check("z", z[..., None], zo[..., None], TOL["bf16"])


def test_favor_workload_full():
    """The random-feature workload at full size, in the launch configuration of the bench."""
    rw = datagen.RF_WORKLOAD
    w = datagen.WORKLOADS[rw["base"]]
    say(f"favor workload {rw['name']}")
    (q, k, v, W), (gfq, gfk), (o, S, z) = _favor(w.B, w.H, w.N, w.d, rw["m"], w.seed, rw["seed"])
    fq, fk = oracle.rf_map(f64(q), f64(W)), oracle.rf_map(f64(k), f64(W))
    check_rf(gfq, fq, "bf16")
    check_rf(gfk, fk, "bf16")
    oo, So, zo, _, _ = oracle.causal(fq, fk, f64(v), mode="identity")
    check("out", o, oo, TOL["bf16"])
    check("S", S, So, TOL["bf16"])


# ---------------------------------------------------------------- random features in one call
def causal_rf(q, k, v, W, flags=0, S0=None, z0=None, chunk=0, seg_len=0):
    B, H, N, d = q.shape
    dv, m = v.shape[-1], W.shape[0]
    out = torch.empty((B, H, N, dv), dtype=q.dtype, device=DEV)
    S = torch.full((B, H, m, dv), float("nan"), device=DEV)
    z = torch.full((B, H, m), float("nan"), device=DEV)
    S0d = None if S0 is None else torch.as_tensor(S0, dtype=torch.float32).to(DEV)
    z0d = None if z0 is None else torch.as_tensor(z0, dtype=torch.float32).to(DEV)
    la().la_causal_fwd_rf(to_dev(q), to_dev(k), to_dev(v), out, to_dev(W), S0d, z0d, S, z,
                          chunk=chunk, seg_len=seg_len, flags=flags)
    torch.cuda.synchronize()
    return f64(out), f64(S), f64(z)


@pytest.mark.parametrize("dtype,d,m,dv,N,seg,flags", [
    ("bf16", 128, 128, 128, 3000, 0, 0), ("bf16", 128, 128, 128, 1000, 192, UNNORM),
    ("bf16", 64, 64, 64, 1111, 0, 0), ("bf16", 64, 64, 64, 65, 0, UNNORM),
    ("bf16", 128, 128, 128, 1, 0, 0), ("bf16", 128, 64, 128, 700, 0, 0),
    ("bf16", 128, 64, 64, 500, 0, 0), ("bf16", 64, 128, 64, 300, 0, 0),
    ("f32", 128, 128, 128, 1000, 0, 0), ("f32", 64, 64, 64, 300, 96, UNNORM),
    ("f32", 32, 16, 32, 200, 0, 0)])
def test_causal_rf(dtype, d, m, dv, N, seg, flags):
    """la_causal_fwd_rf against the oracle's features and recurrence, with a carried initial
    state: bf16 with m == d == d_v maps inside the attention kernels, other shapes and float32
    go through memory (float32 with m == d_v in {64, 128}: then the float32 matrix-core kernels)."""
    q, k, v = datagen.qkv(2, 2, N, d, dv, 1500 + d + m + N, 1 / math.sqrt(d), dtype)
    W = datagen.projections(m, d, 1600 + m, dtype)
    fq, fk = oracle.rf_map(f64(q), f64(W)), oracle.rf_map(f64(k), f64(W))
    mode, norm = MODE[IDENT | flags]
    # a carried state from 64 earlier tokens
    qp, kp, vp = datagen.qkv(2, 2, 64, d, dv, 1700 + d, 1 / math.sqrt(d), dtype)
    _, S0, z0, _, _ = oracle.causal(oracle.rf_map(f64(qp), f64(W)), oracle.rf_map(f64(kp), f64(W)),
                                    f64(vp), mode="identity")
    S0, z0 = S0.astype(np.float32), z0.astype(np.float32)
    say(f"causal rf dtype={dtype} d={d} m={m} dv={dv} N={N} seg={seg} flags={flags}")
    o, S, z = causal_rf(q, k, v, W, flags=flags, S0=S0, z0=z0, seg_len=seg)
    oo, So, zo, _, _ = oracle.causal(fq, fk, f64(v), S0=S0, z0=z0, mode=mode, normalize=norm)
    check("out", o, oo, TOL[dtype])
    check("S", S, So, TOL[dtype])
    check("z", z, zo, TOL[dtype])


def test_causal_rf_fused_equals_two_pass():
    """The map inside the staging gives the features the separate feature kernel writes, so
    the one-call form and the two-pass form agree to far below the bf16 tolerance."""
    q, k, v = datagen.qkv(2, 4, 2500, 128, 128, 1801, 1 / math.sqrt(128), "bf16")
    W = datagen.projections(128, 128, 1802, "bf16")
    say("causal rf fused vs two-pass")
    o1, S1, z1 = causal_rf(q, k, v, W)
    fq, fk = rf_gpu(q, W), rf_gpu(k, W)
    o2, S2, z2 = causal_ex(fq, fk, v, IDENT)
    check("out", o1, o2, 1e-3)
    check("S", S1, S2, 1e-5)
    check("z", z1, z2, 1e-5)


def test_causal_rf_workload_full():
    """The random-feature workload in one call, in the launch configuration of the bench."""
    rw = datagen.RF_WORKLOAD
    w = datagen.WORKLOADS[rw["base"]]
    q, k, v = datagen.qkv(w.B, w.H, w.N, w.d, w.dv, w.seed, w.scale, "bf16")
    W = datagen.projections(rw["m"], w.d, rw["seed"], "bf16")
    say(f"causal rf workload {rw['name']}")
    o, S, z = causal_rf(q, k, v, W)
    fq, fk = oracle.rf_map(f64(q), f64(W)), oracle.rf_map(f64(k), f64(W))
    oo, So, zo, _, _ = oracle.causal(fq, fk, f64(v), mode="identity")
    check("out", o, oo, TOL["bf16"])
    check("S", S, So, TOL["bf16"])
