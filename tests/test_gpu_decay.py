"""GPU parity of the decayed recurrence (la_causal_fwd_decay, la_decode_step_decay) against
the float64 oracle with the same per-head gamma.

Criteria as for the base forms: row-wise max-norm relative error within 1e-5 (float32) and
2e-2 (bfloat16); the hand-derived example to one rounding of the output dtype. The retention
form (identity map, no division) on signed q and k sums terms that can cancel (with gamma = 0
a row is (q_t . k_t) v_t, and q_t . k_t can be far smaller than its terms): for float32 there
the error of each row is measured against the same sums over absolute values (check_bounded),
the scale float32 rounding error is proportional to. bfloat16 keeps the row-wise check.
"""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import DEV, check, check_bounded, f64, la, say, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
EXACT_TOL = {"f32": 2e-7, "bf16": 2.0 ** -8}
IDENT, UNNORM = 1, 2
MODE = {0: ("elu1", True), IDENT: ("identity", True), UNNORM: ("elu1", False),
        IDENT | UNNORM: ("identity", False)}


def causal_decay(q, k, v, gamma, flags, S0=None, z0=None, chunk=0, seg_len=0):
    B, H, N, d = q.shape
    dv = v.shape[-1]
    out = torch.empty((B, H, N, dv), dtype=q.dtype, device=DEV)
    S = torch.full((B, H, d, dv), float("nan"), device=DEV)
    z = torch.full((B, H, d), float("nan"), device=DEV)
    S0d = None if S0 is None else torch.as_tensor(S0, dtype=torch.float32).to(DEV)
    z0d = None if z0 is None else torch.as_tensor(z0, dtype=torch.float32).to(DEV)
    g = torch.as_tensor(gamma, dtype=torch.float32).to(DEV)
    la().la_causal_fwd_decay(to_dev(q), to_dev(k), to_dev(v), out, g, S0d, z0d, S, z, chunk=chunk,
                             seg_len=seg_len, flags=flags)
    torch.cuda.synchronize()
    return f64(out), f64(S), f64(z)


def _feat(rows, d, dtype):
    rows = np.asarray(rows, dtype=np.float64)
    out = np.zeros((1, 1, rows.shape[0], d))
    out[0, 0, :, : rows.shape[1]] = rows
    return torch.from_numpy(out).to(datagen.DTYPES[dtype])


@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 128, 0), ("bf16", 64, 0), ("f32", 16, 16),
                                           ("bf16", 32, 32), ("f32", 128, 0)])
def test_decay_worked_example(golden, dtype, d, chunk):
    """The hand-derived gamma = 0.5 example: causal outputs, S3, z3, and the three reads of
    S3 as decode steps, in the retention form (identity map, no division)."""
    g = golden("w8_decay_derived.json")
    dr = g["derived"]
    k, v = _feat(g["k"], d, dtype), _feat(g["v"], d, dtype)
    say(f"decay example dtype={dtype} d={d} chunk={chunk}")
    o, S, z = causal_decay(k, k, v, [g["gamma"]], IDENT | UNNORM, chunk=chunk)
    want = np.zeros((1, 1, 3, d))
    want[0, 0, :, :2] = dr["causal_outputs_unnormalised_q_equal_k"]
    check("outputs", o, want, EXACT_TOL[dtype])
    Sw = np.zeros((1, 1, d, d))
    Sw[0, 0, :2, :2] = dr["S3"]
    check("S3", S, Sw, 1e-6)
    zw = np.zeros((1, 1, d))
    zw[0, 0, :2] = dr["z3"]
    check("z3", z, zw, 1e-6)
    gam = torch.tensor([g["gamma"]], dtype=torch.float32, device=DEV)
    for qs, key in (([1, 0], "q=[1,0]"), ([0, 1], "q=[0,1]"), ([1, 1], "q=[1,1]")):
        Sd = torch.zeros((1, 1, d, d), device=DEV)
        zd = torch.zeros((1, 1, d), device=DEV)
        for t in range(3):
            qrow = qs if t == 2 else g["k"][t]
            qt = to_dev(_feat([qrow], d, dtype)[:, :, 0])
            kt = to_dev(_feat([g["k"][t]], d, dtype)[:, :, 0])
            vt = to_dev(_feat([g["v"][t]], d, dtype)[:, :, 0])
            out = torch.empty((1, 1, d), dtype=kt.dtype, device=DEV)
            la().la_decode_step_decay(qt, kt, vt, out, Sd, zd, gam, flags=IDENT | UNNORM)
        torch.cuda.synchronize()
        want = np.zeros((1, 1, d))
        want[0, 0, :2] = dr["reads_unnormalised"][key]
        check(f"decode read {key}", f64(out), want, EXACT_TOL[dtype])


GAMMAS = [0.9, 0.5, 1.0, 0.0, 0.99]


@pytest.mark.parametrize("flags", [0, UNNORM, IDENT | UNNORM])
@pytest.mark.parametrize("dtype,d,chunk,seg", [("bf16", 128, 0, 0), ("bf16", 128, 0, 128),
                                               ("bf16", 64, 0, 192), ("f32", 32, 16, 0),
                                               ("bf16", 16, 32, 96), ("f32", 64, 32, 64),
                                               ("f32", 128, 0, 0), ("f32", 128, 0, 96)])
def test_decay_causal(flags, dtype, d, chunk, seg):
    """Per-head gamma including 0 and 1, a carried initial state, several segments (the
    decayed scan) and a ragged tail."""
    B, H, N = 2, len(GAMMAS), 700 + d
    q, k, v = datagen.qkv(B, H, N, d, d, 900 + d + flags, 1 / math.sqrt(d), dtype)
    mode, norm = MODE[flags]
    n1 = 157
    say(f"decay causal flags={flags} dtype={dtype} d={d} chunk={chunk} seg={seg}")
    _, S1, z1, _, _ = oracle.causal(f64(q[:, :, :n1]), f64(k[:, :, :n1]), f64(v[:, :, :n1]),
                                    mode=mode, normalize=norm, gamma=GAMMAS)
    S1, z1 = S1.astype(np.float32), z1.astype(np.float32)
    qb, kb, vb = (x[:, :, n1:].contiguous() for x in (q, k, v))
    o, S, z = causal_decay(qb, kb, vb, GAMMAS, flags, S0=S1, z0=z1, chunk=chunk, seg_len=seg)
    oo, So, zo, _, _ = oracle.causal(f64(qb), f64(kb), f64(vb), S0=S1, z0=z1, mode=mode,
                                     normalize=norm, gamma=GAMMAS)
    if flags == IDENT | UNNORM and dtype == "f32":
        # signed features: rows may cancel; bound each row by the sums over |q|, |k|, |v|
        ab = [np.abs(f64(x)) for x in (q, k, v)]
        ob, Sb, zb, _, _ = oracle.causal(*ab, mode=mode, normalize=norm, gamma=GAMMAS)
        check_bounded("out", o, oo, ob[:, :, n1:], TOL[dtype])
        check_bounded("S", S, So, Sb, TOL[dtype])
        check_bounded("z", z, zo, zb, TOL[dtype])
        return
    check("out", o, oo, TOL[dtype])
    check("S", S, So, TOL[dtype])
    check("z", z, zo, TOL[dtype])   # rows = heads


@pytest.mark.parametrize("flags", [0, IDENT | UNNORM])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 32), ("bf16", 64), ("f32", 128)])
def test_decay_decode_chain(flags, dtype, d):
    """Prefill of N tokens, then decode steps, equals the causal form over all tokens."""
    B, H, N, steps = 2, len(GAMMAS), 300, 3
    q, k, v = datagen.qkv(B, H, N + steps, d, d, 950 + d + flags, 1 / math.sqrt(d), dtype)
    mode, norm = MODE[flags]
    say(f"decay decode chain flags={flags} dtype={dtype} d={d}")
    pre = [x[:, :, :N].contiguous() for x in (q, k, v)]
    _, S, z = causal_decay(*pre, GAMMAS, flags)
    Sd = torch.from_numpy(S.astype(np.float32)).to(DEV)
    zd = torch.from_numpy(z.astype(np.float32)).to(DEV)
    gam = torch.tensor(GAMMAS, dtype=torch.float32, device=DEV)
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v), mode=mode, normalize=norm,
                                     gamma=GAMMAS)
    signed = flags == IDENT | UNNORM and dtype == "f32"
    if signed:
        ob, Sb, zb, _, _ = oracle.causal(*[np.abs(f64(x)) for x in (q, k, v)], mode=mode,
                                         normalize=norm, gamma=GAMMAS)
    for t in range(N, N + steps):
        qt, kt, vt = (to_dev(x[:, :, t].contiguous()) for x in (q, k, v))
        out = torch.empty((B, H, d), dtype=qt.dtype, device=DEV)
        la().la_decode_step_decay(qt, kt, vt, out, Sd, zd, gam, flags=flags)
        torch.cuda.synchronize()
        if signed:
            check_bounded(f"step {t}", f64(out), oo[:, :, t], ob[:, :, t], TOL[dtype])
        else:
            check(f"step {t}", f64(out), oo[:, :, t], TOL[dtype])
    if signed:
        check_bounded("S", f64(Sd), So, Sb, TOL[dtype])
        check_bounded("z", f64(zd), zo, zb, TOL[dtype])
    else:
        check("S", f64(Sd), So, TOL[dtype])
        check("z", f64(zd), zo, TOL[dtype])


@pytest.mark.parametrize("d,seg", [(128, 0), (64, 96), (32, 0)])
def test_retention_float32_rowwise(d, seg):
    """The float32 retention form (identity map, no division, per-head decay) with positive q,
    k and v: no row can cancel, so the plain row-wise bar of 1e-5 applies (the signed cases
    above are bounded by their absolute-value sums instead). d = 128, 64 run the float32
    matrix-core kernels, d = 32 the vector-ALU ones."""
    B, H, N = 2, len(GAMMAS), 900 + d
    q = datagen.positive((B, H, N, d), 980 + d, 1 / math.sqrt(d), "f32")
    k = datagen.positive((B, H, N, d), 981 + d, 1 / math.sqrt(d), "f32")
    v = datagen.positive((B, H, N, d), 982 + d, 1.0, "f32")
    say(f"float32 retention, positive inputs, d={d} seg={seg}")
    o, S, z = causal_decay(q, k, v, GAMMAS, IDENT | UNNORM, seg_len=seg)
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v), mode="identity", normalize=False,
                                     gamma=GAMMAS)
    check("out", o, oo, TOL["f32"])
    check("S", S, So, TOL["f32"])
    check("z", z, zo, TOL["f32"])


def test_decay_one_equals_base():
    """gamma = 1 for every head gives the undecayed form (within rounding of the decay path)."""
    q, k, v = datagen.qkv(1, 4, 1500, 128, 128, 971, 1 / math.sqrt(128), "bf16")
    say("decay 1 vs base")
    o, S, z = causal_decay(q, k, v, [1.0] * 4, 0)
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v))
    check("out", o, oo, TOL["bf16"])
    check("S", S, So, TOL["bf16"])


def test_retention_workload_full():
    """The retention form at the full causal workload (B=2 H=16 N=8192 d=128), per-head
    decays 1 - 2^-(5+h), in the launch configuration of the bench."""
    rw = datagen.DECAY_WORKLOAD
    w = datagen.WORKLOADS[rw["base"]]
    q, k, v = datagen.qkv(w.B, w.H, w.N, w.d, w.dv, w.seed, w.scale, "bf16")
    gam = datagen.decay_rates(w.H).numpy()
    say(f"retention workload {rw['name']}")
    o, S, z = causal_decay(q, k, v, gam, IDENT | UNNORM)
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v), mode="identity", normalize=False,
                                     gamma=gam.astype(np.float64))
    check("out", o, oo, TOL["bf16"])
    check("S", S, So, TOL["bf16"])


@pytest.mark.parametrize("dtype,d,chunk,seg", [("bf16", 128, 0, 64), ("f32", 32, 16, 0),
                                               ("f32", 128, 0, 64)])
def test_decay_out_of_range_is_nan(dtype, d, chunk, seg):
    """A negative or NaN gamma (outside the [0, 1] contract) makes every output and the state
    of its head NaN, in the prefill and in the decode step alike; the other heads are
    unaffected."""
    gam = [0.9, -0.5, float("nan"), 0.5]
    good = [0, 3]
    B, H, N = 2, len(gam), 300
    q, k, v = datagen.qkv(B, H, N + 1, d, d, 990 + d, 1 / math.sqrt(d), dtype)
    pre = [x[:, :, :N].contiguous() for x in (q, k, v)]
    say(f"decay out of range dtype={dtype} d={d} chunk={chunk} seg={seg}")
    o, S, z = causal_decay(*pre, gam, 0, chunk=chunk, seg_len=seg)
    for h in (1, 2):
        assert np.isnan(o[:, h]).all() and np.isnan(S[:, h]).all() and np.isnan(z[:, h]).all(), h
    sub = [f64(x[:, good]) for x in pre]
    oo, So, zo, _, _ = oracle.causal(*sub, gamma=[gam[h] for h in good])
    check("good heads out", o[:, good], oo, TOL[dtype])
    check("good heads S", S[:, good], So, TOL[dtype])
    # one decode step from the prefill's state
    Sd = torch.from_numpy(S.astype(np.float32)).to(DEV)
    zd = torch.from_numpy(z.astype(np.float32)).to(DEV)
    qt, kt, vt = (to_dev(x[:, :, N].contiguous()) for x in (q, k, v))
    out = torch.empty((B, H, d), dtype=qt.dtype, device=DEV)
    la().la_decode_step_decay(qt, kt, vt, out, Sd, zd, torch.tensor(gam, dtype=torch.float32,
                                                                     device=DEV))
    torch.cuda.synchronize()
    od, Sn = f64(out), f64(Sd)
    for h in (1, 2):
        assert np.isnan(od[:, h]).all() and np.isnan(Sn[:, h]).all(), h
    oo2, So2, _, _, _ = oracle.causal(*[f64(x[:, good]) for x in (q, k, v)],
                                      gamma=[gam[h] for h in good])
    check("good heads decode", od[:, good], oo2[:, :, N], TOL[dtype])
    check("good heads decode S", Sn[:, good], So2, TOL[dtype])
