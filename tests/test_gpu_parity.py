"""GPU parity: the HIP path, called through the C ABI, against the float64 oracle.

Criterion: row-wise max-norm relative error (oracle/compare.py) within 1e-5 for float32 inputs
and 2e-2 for bfloat16 inputs; the pages' worked examples, embedded in the supported head
sizes, are checked to one rounding of the output dtype.
"""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import causal, check, f64, global_, say, to_dev, DEV, la

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
# one rounding of the output dtype (worked examples with exact inputs)
EXACT_TOL = {"f32": 2e-7, "bf16": 2.0 ** -8}
RAW = {0: -1000.0, 1: 0.0, 3: 2.0}   # raw inputs whose ELU+1 features are 0, 1, 3

# (dtype, d, chunk): the matrix-core kernel (bf16, d in {64,128}, chunk 64) and the
# vector-ALU kernel (chunks 16/32, either dtype)
PATHS = [("f32", 16, 16), ("f32", 16, 32), ("bf16", 16, 32), ("bf16", 64, 64),
         ("bf16", 128, 64), ("f32", 128, 32), ("bf16", 128, 16)]


def _embed_feat(rows, d):
    """Feature rows (0/1/3 values, width <= d) -> raw [1,1,N,d] inputs, padding feature 0."""
    rows = np.asarray(rows, dtype=np.float64)
    out = np.full((1, 1, rows.shape[0], d), RAW[0])
    for i in range(rows.shape[0]):
        for j in range(rows.shape[1]):
            out[0, 0, i, j] = RAW[int(rows[i, j])]
    return out


def _embed_val(rows, dv):
    rows = np.asarray(rows, dtype=np.float64)
    out = np.zeros((1, 1, rows.shape[0], dv))
    out[0, 0, :, : rows.shape[1]] = rows
    return out


def _t(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(datagen.DTYPES[dtype])


@pytest.mark.parametrize("dtype,d,chunk", PATHS)
def test_worked_examples_causal(golden, dtype, d, chunk):
    """Two-token read (10/3) and the three-token example, through ELU+1, on the GPU."""
    g1 = golden("w1_two_token_read.json")
    q1 = np.array(g1["q_at_position_1"], float)
    q = _t(_embed_feat(np.stack([q1, q1]), d), dtype)
    k = _t(_embed_feat(g1["k"], d), dtype)
    v = _t(_embed_val(g1["v"], d), dtype)
    say(f"W1 two-token read dtype={dtype} d={d} chunk={chunk}")
    o, S, z = causal(q, k, v, chunk=chunk)
    want = np.zeros((1, 1, 2, d))
    want[0, 0, :, 0] = [g1["derived"]["output_at_position_0"], 10.0 / 3.0]
    check("W1 out", o, want, EXACT_TOL[dtype])
    Sw = np.zeros((1, 1, d, d))
    Sw[0, 0, :2, 0] = np.array(g1["printed"]["S_after_token_1"], float)[:, 0]
    check("W1 S", S, Sw, 1e-6)
    zw = np.zeros((1, 1, d))
    zw[0, 0, :2] = g1["printed"]["z_after_token_1"]
    check("W1 z", z[..., None], zw[..., None], 1e-6)

    g2 = golden("w2_three_token.json")
    k = _t(_embed_feat(g2["k"], d), dtype)
    v = _t(_embed_val(g2["v"], d), dtype)
    say(f"W2 three-token dtype={dtype} d={d} chunk={chunk}")
    o, S, z = causal(k, k, v, chunk=chunk)
    want = _embed_val(g2["derived"]["causal_outputs_with_q_equal_k"], d)
    check("W2 out", o, want, EXACT_TOL[dtype])
    Sw = np.zeros((1, 1, d, d))
    Sw[0, 0, :2, :2] = g2["printed"]["S3"]
    check("W2 S", S, Sw, 1e-6)


@pytest.mark.parametrize("dtype,d,chunk", PATHS)
def test_worked_example_global(golden, dtype, d, chunk):
    g = golden("w6_global_example.json")
    q = _t(_embed_feat(g["q"], d), dtype)
    k = _t(_embed_feat(g["k"], d), dtype)
    v = _t(_embed_val(g["v"], d), dtype)
    say(f"W6 global dtype={dtype} d={d} chunk={chunk}")
    o, S, z = global_(q, k, v, chunk=chunk)
    check("W6 out", o, _embed_val(g["derived"]["global_outputs"], d), EXACT_TOL[dtype])
    Sw = np.zeros((1, 1, d, d))
    Sw[0, 0, :2, :2] = g["printed_state"]["S"]
    check("W6 S", S, Sw, 1e-6)


@pytest.mark.parametrize("dtype,d", [("f32", 16), ("bf16", 16), ("bf16", 128), ("f32", 128)])
def test_worked_example_decode(golden, dtype, d):
    """The decode example: two steps from the zero state; phi(q) = [3, 1] -> [0.75, 0.5]."""
    g = golden("w3_decode_example.json")
    S = torch.zeros((1, 1, d, d), dtype=torch.float32, device=DEV)
    z = torch.zeros((1, 1, d), dtype=torch.float32, device=DEV)
    qr = to_dev(_t(_embed_feat([g["phi_q"]], d)[:, :, 0], dtype))
    for t in range(2):
        kr = to_dev(_t(_embed_feat([g["phi_k"][t]], d)[:, :, 0], dtype))
        vr = to_dev(_t(_embed_val([g["v"][t]], d)[:, :, 0], dtype))
        out = torch.empty((1, 1, d), dtype=kr.dtype, device=DEV)
        say(f"W3 decode step {t} dtype={dtype} d={d}")
        la().la_decode_step(qr, kr, vr, out, S, z)
    torch.cuda.synchronize()
    want = np.zeros((1, 1, d))
    want[0, 0, :2] = g["printed"]["output"]
    check("W3 out", f64(out), want, EXACT_TOL[dtype])
    Sw = np.zeros((1, 1, d, d))
    Sw[0, 0, :2, :2] = g["printed"]["S"]
    check("W3 S", f64(S), Sw, 1e-7)


# ---------------------------------------------------------------- the five workloads
def _workload(n):
    w = datagen.WORKLOADS[n]
    q, k, v = datagen.qkv(w.B, w.H, w.N, w.d, w.dv, w.seed, w.scale, w.dtype)
    return w, q, k, v


@pytest.mark.parametrize("chunk,seg", [(0, 0), (16, 0), (32, 0), (64, 0), (128, 0), (16, 16),
                                       (16, 32), (32, 32)])
def test_workload1_causal_f32(chunk, seg):
    w, q, k, v = _workload(1)
    say(f"workload 1 {w.name} chunk={chunk} seg_len={seg}")
    o, S, z = causal(q, k, v, chunk=chunk, seg_len=seg)
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v))
    check("out", o, oo, TOL["f32"])
    check("S", S, So, TOL["f32"])
    check("z", z[..., None], zo[..., None], TOL["f32"])


@pytest.mark.parametrize("chunk,seg", [(64, 0), (64, 64), (64, 2048), (32, 0)])
def test_workload2_causal(chunk, seg):
    w, q, k, v = _workload(2)
    say(f"workload 2 {w.name} chunk={chunk} seg_len={seg}")
    o, S, z = causal(q, k, v, chunk=chunk, seg_len=seg)
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v))
    check("out", o, oo, TOL["bf16"])
    check("S", S, So, TOL["bf16"])
    check("z", z[..., None], zo[..., None], TOL["bf16"])


def test_workload3_causal_full():
    w, q, k, v = _workload(3)
    say(f"workload 3 {w.name} (launch configuration of the bench)")
    o, S, z = causal(q, k, v)
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v))
    check("out", o, oo, TOL["bf16"])
    check("S", S, So, TOL["bf16"])
    check("z", z[..., None], zo[..., None], TOL["bf16"])


def test_workload4_global_full():
    """The global workload (B=1 H=8 N=100000 d=128) in the bench's launch configuration: every
    one of the 800,000 output rows (including the ragged last 32 of each head), S and z."""
    w, q, k, v = _workload(4)
    say(f"workload 4 {w.name}")
    o, S, z = global_(q, k, v)
    oo, So, zo, _, _ = oracle.global_(f64(q), f64(k), f64(v))
    check("out (all rows)", o, oo, TOL["bf16"])
    check("out (last 32 rows of each head)", o[:, :, -32:], oo[:, :, -32:], TOL["bf16"])
    check("S", S, So, TOL["bf16"])
    check("z", z[..., None], zo[..., None], TOL["bf16"])


def test_global_d64_many_segments():
    """The d = 64 global form with several segments per head (segment sums, their total) and the
    read's own split of the sequence, with a ragged tail: every output row against the oracle."""
    q, k, v = datagen.qkv(2, 4, 20011, 64, 64, 4242, 1 / 8, "bf16")
    say("global d=64 B=2 H=4 N=20011")
    o, S, z = global_(q, k, v)
    oo, So, zo, _, _ = oracle.global_(f64(q), f64(k), f64(v))
    check("out", o, oo, TOL["bf16"])
    check("S", S, So, TOL["bf16"])
    check("z", z[..., None], zo[..., None], TOL["bf16"])


def _decode_run(B, H, d, prior, steps, seed):
    """Seeded prior tokens -> oracle state (float64, rounded to float32) -> `steps` decode
    steps on the GPU and in the oracle."""
    kp, vp = datagen.qkv(B, H, prior, d, d, seed, 1 / math.sqrt(d), "bf16")[1:]
    _, S0, z0, _, _ = oracle.global_(None, f64(kp), f64(vp))
    S0 = S0.astype(np.float32)
    z0 = z0.astype(np.float32)
    S = torch.from_numpy(S0).to(DEV)
    z = torch.from_numpy(z0).to(DEV)
    So, zo = S0.astype(np.float64), z0.astype(np.float64)
    toks = datagen.qkv(B, H, steps, d, d, seed + 1, 1 / math.sqrt(d), "bf16")
    for t in range(steps):
        q, k, v = (x[:, :, t].contiguous() for x in toks)
        out = torch.empty((B, H, d), dtype=torch.bfloat16, device=DEV)
        say(f"decode B={B} H={H} d={d} prior={prior} step {t}")
        la().la_decode_step(to_dev(q), to_dev(k), to_dev(v), out, S, z)
        torch.cuda.synchronize()
        oo, So, zo = oracle.decode_step(f64(q), f64(k), f64(v), So, zo)
        check(f"out step {t}", f64(out), oo, TOL["bf16"])
    check("S", f64(S), So, 1e-6)
    check("z", f64(z)[..., None], zo[..., None], 1e-6)


@pytest.mark.timeout(900)
def test_workload5_decode_bench_configuration():
    """The decode workload exactly as the bench runs it: 256 x 32 heads, a starting state built
    by the library's global form from the seeded 4096-token prior of every head, then 1000
    decode steps of fresh tokens, the state updated in place. Against the oracle (its own
    starting state from the same prior, then the recurrence over the 1000 step tokens): the
    starting state of every head; the outputs of every head at every step (so every head at the
    last step, and the 256-head sample below at steps 1, 10 and 100); the state after 1, 10, 100
    and 1000 steps on a 256-head sample; and the final state of every head."""
    w = datagen.WORKLOADS[5]
    B, H, d, steps = w.B, w.H, w.d, w.steps
    m = la()
    S = torch.empty(B, H, d, d, device=DEV)
    z = torch.empty(B, H, d, device=DEV)
    blocks = []
    say(f"decode workload {w.name}: prior states ({B // datagen.DECODE_PRIOR_BLOCK} blocks)")
    for b0 in range(0, B, datagen.DECODE_PRIOR_BLOCK):
        kp, vp = datagen.decode_prior(w, b0)
        n = kp.shape[0]
        m.la_global_fwd(None, kp, vp, None, S[b0:b0 + n], z[b0:b0 + n])
        _, So, zo, _, _ = oracle.global_(None, f64(kp), f64(vp))
        del kp, vp
        torch.cuda.synchronize()
        check(f"prior S rows {b0}..{b0 + n - 1}", f64(S[b0:b0 + n]), So, TOL["bf16"])
        check(f"prior z rows {b0}..{b0 + n - 1}", f64(z[b0:b0 + n])[..., None], zo[..., None],
              TOL["bf16"])
        blocks.append((b0, n, So, zo))
    # 256-head sample (fixed seed): (batch row, head) pairs
    rng = np.random.default_rng(5)
    sample = np.sort(rng.choice(B * H, 256, replace=False))
    sb, sh = sample // H, sample % H
    sbd, shd = torch.from_numpy(sb).to(DEV), torch.from_numpy(sh).to(DEV)
    snaps = {}
    toks = datagen.decode_tokens(w, steps)
    outs = torch.empty(steps, B, H, d, dtype=torch.bfloat16, device=DEV)
    say(f"decode workload {w.name}: {steps} steps on the GPU")
    for t in range(steps):
        m.la_decode_step(toks[0][t], toks[1][t], toks[2][t], outs[t], S, z)
        if t + 1 in (1, 10, 100):
            snaps[t + 1] = (S[sbd, shd].clone(), z[sbd, shd].clone())
    torch.cuda.synchronize()
    snaps[steps] = (S[sbd, shd].clone(), z[sbd, shd].clone())
    # the oracle, one block of batch rows at a time: the recurrence over the step tokens from the
    # oracle's own starting state
    Ssamp = {}
    for b0, n, So, zo in blocks:
        qs, ks, vs = (f64(x[:, b0:b0 + n].permute(1, 2, 0, 3).contiguous()) for x in toks)
        oo, Sn, zn, _, _ = oracle.causal(qs, ks, vs, S0=So, z0=zo)
        got = f64(outs[:, b0:b0 + n].permute(1, 2, 0, 3).contiguous())
        say(f"  rows {b0}..{b0 + n - 1}")
        check(f"outs rows {b0}..{b0 + n - 1} (all steps)", got, oo, TOL["bf16"])
        check(f"out at step {steps}", got[:, :, -1], oo[:, :, -1], TOL["bf16"])
        check(f"final S rows {b0}..{b0 + n - 1}", f64(S[b0:b0 + n]), Sn, TOL["bf16"])
        check(f"final z rows {b0}..{b0 + n - 1}", f64(z[b0:b0 + n])[..., None], zn[..., None],
              TOL["bf16"])
        # the sampled heads of this block: state after 1, 10, 100 steps
        sel = np.nonzero((sb >= b0) & (sb < b0 + n))[0]
        if sel.size == 0:
            continue
        for t in (1, 10, 100):
            _, St, zt, _, _ = oracle.causal(qs[sb[sel] - b0, sh[sel]][None, :, :t],
                                            ks[sb[sel] - b0, sh[sel]][None, :, :t],
                                            vs[sb[sel] - b0, sh[sel]][None, :, :t],
                                            S0=So[sb[sel] - b0, sh[sel]][None],
                                            z0=zo[sb[sel] - b0, sh[sel]][None])
            Ssamp.setdefault(t, []).append((sel, St[0], zt[0]))
        Ssamp.setdefault(steps, []).append((sel, Sn[sb[sel] - b0, sh[sel]], zn[sb[sel] - b0, sh[sel]]))
    for t, parts in Ssamp.items():
        Sw = np.empty((256, d, d))
        zw = np.empty((256, d))
        for sel, St, zt in parts:
            Sw[sel] = St
            zw[sel] = zt
        check(f"sampled S after {t} steps", f64(snaps[t][0]), Sw, TOL["bf16"])
        check(f"sampled z after {t} steps", f64(snaps[t][1])[..., None], zw[..., None], TOL["bf16"])


def test_workload5_decode_full_prior_float32_state():
    """The decode workload's 4096-token prior on 64 of its heads, starting from the oracle's
    state rounded to float32 (so the state itself is checked at float32 precision)."""
    w = datagen.WORKLOADS[5]
    _decode_run(2, w.H, w.d, prior=w.prior, steps=2, seed=w.seed + 10)


# ---------------------------------------------------------------- edges and invariants
@pytest.mark.parametrize("dtype,d,dv,N,chunk", [
    ("bf16", 128, 128, 1, 0), ("bf16", 128, 128, 63, 0), ("bf16", 128, 128, 65, 0),
    ("bf16", 128, 128, 1000, 0), ("bf16", 64, 64, 1, 0), ("bf16", 64, 64, 129, 0),
    ("f32", 128, 128, 65, 16), ("f32", 64, 32, 77, 32), ("bf16", 32, 128, 50, 0),
    ("bf16", 128, 16, 50, 0), ("f32", 16, 16, 1, 0), ("bf16", 16, 64, 300, 16),
    ("f32", 32, 32, 300, 128), ("bf16", 16, 16, 1000, 128), ("f32", 64, 64, 333, 64),
    ("bf16", 64, 128, 200, 64)])
def test_ragged_and_mixed_shapes(dtype, d, dv, N, chunk):
    q, k, v = datagen.qkv(2, 3, N, d, dv, 77 + N, 1 / math.sqrt(d), dtype)
    say(f"ragged dtype={dtype} d={d} dv={dv} N={N} chunk={chunk}")
    o, S, z = causal(q, k, v, chunk=chunk)
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v))
    check("out", o, oo, TOL[dtype])
    check("S", S, So, TOL[dtype])
    og, Sg, zg = global_(q, k, v, chunk=chunk)
    oo, So, zo, _, _ = oracle.global_(f64(q), f64(k), f64(v))
    check("global out", og, oo, TOL[dtype])
    check("global S", Sg, So, TOL[dtype])


@pytest.mark.parametrize("seg", [64, 128, 512, 1024, 4096])
def test_segment_split_sweep(seg):
    """Results do not depend on how the sequence is split across workgroups."""
    q, k, v = datagen.qkv(1, 4, 4096 + 40, 128, 128, 5, 1 / math.sqrt(128), "bf16")
    say(f"segment sweep seg_len={seg}")
    o, S, z = causal(q, k, v, seg_len=seg)
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v))
    check("out", o, oo, TOL["bf16"])
    check("S", S, So, TOL["bf16"])


@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 128, 0), ("bf16", 64, 0), ("f32", 32, 16)])
def test_state_carry_split(dtype, d, chunk):
    """Causal over [0, N) equals [0, N1) then [N1, N) with the state carried through S, z,
    and a prefill followed by one decode step equals causal over N + 1 at position N."""
    N, n1 = 700, 333
    q, k, v = datagen.qkv(2, 2, N + 1, d, d, 9, 1 / math.sqrt(d), dtype)
    qa, ka, va = (x[:, :, :n1].contiguous() for x in (q, k, v))
    qb, kb, vb = (x[:, :, n1:N].contiguous() for x in (q, k, v))
    say(f"state carry dtype={dtype} d={d}")
    oa, Sa, za = causal(qa, ka, va, chunk=chunk)
    ob, Sb, zb = causal(qb, kb, vb, S0=Sa.astype(np.float32), z0=za.astype(np.float32), chunk=chunk)
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v))
    check("two-piece out", np.concatenate([oa, ob], axis=2), oo[:, :, :N], TOL[dtype])
    _, Sn, zn, _, _ = oracle.causal(f64(q[:, :, :N]), f64(k[:, :, :N]), f64(v[:, :, :N]))
    check("two-piece S", Sb, Sn, TOL[dtype])
    S = torch.from_numpy(Sb.astype(np.float32)).to(DEV)
    z = torch.from_numpy(zb.astype(np.float32)).to(DEV)
    out = torch.empty((2, 2, 1, d), dtype=q.dtype, device=DEV)
    la().la_decode_step(to_dev(q[:, :, N:]), to_dev(k[:, :, N:]), to_dev(v[:, :, N:]), out, S, z)
    torch.cuda.synchronize()
    check("prefill+decode", f64(out), oo[:, :, N:], TOL[dtype])


@pytest.mark.parametrize("decay", [False, True])
@pytest.mark.parametrize("B,H,N,seg", [(4, 16, 4096, 256), (3, 3, 2000, 128), (1, 8, 1000, 64)])
def test_initial_state_in_place_segments(B, H, N, seg, decay):
    """The initial state passed in S, z, which also receive the final state, with many
    segments: 1,024 workgroups in the first case, more than the chip runs at once, so a head's
    last segment may finish (and write the final state) before a later-dispatched segment of
    the same head starts; every segment must still start from the initial state. B*H = 9
    takes the plain block order, 64 and 8 the order that keeps a head's segments on one XCD."""
    d, n0 = 128, 50
    q, k, v = datagen.qkv(B, H, N + n0, d, d, 2100 + B * H + N, 1 / math.sqrt(d), "bf16")
    gamma = np.linspace(0.9, 1.0, H) if decay else None
    _, S0, z0, _, _ = oracle.causal(f64(q[:, :, :n0]), f64(k[:, :, :n0]), f64(v[:, :, :n0]),
                                    gamma=gamma)
    S0, z0 = S0.astype(np.float32), z0.astype(np.float32)
    qb, kb, vb = (x[:, :, n0:].contiguous() for x in (q, k, v))
    say(f"initial state in place B={B} H={H} N={N} seg_len={seg} decay={decay}")
    out = torch.empty((B, H, N, d), dtype=qb.dtype, device=DEV)
    S, z = torch.from_numpy(S0).to(DEV), torch.from_numpy(z0).to(DEV)
    if decay:
        g = torch.from_numpy(gamma.astype(np.float32)).to(DEV)
        la().la_causal_fwd_decay(to_dev(qb), to_dev(kb), to_dev(vb), out, g, S, z, S, z,
                                 seg_len=seg)
    else:
        la().la_causal_fwd(to_dev(qb), to_dev(kb), to_dev(vb), out, S, z, seg_len=seg)
    torch.cuda.synchronize()
    oo, So, zo, _, _ = oracle.causal(f64(qb), f64(kb), f64(vb), S0=S0, z0=z0, gamma=gamma)
    check("out", f64(out), oo, TOL["bf16"])
    check("S", f64(S), So, TOL["bf16"])
    check("z", f64(z), zo, TOL["bf16"])


def test_bit_reproducible():
    """Fixed reduction order: two runs give identical bytes (causal, global, decode)."""
    q, k, v = datagen.qkv(2, 8, 3000, 128, 128, 21, 1 / math.sqrt(128), "bf16")
    say("reproducibility")
    a = causal(q, k, v)
    b = causal(q, k, v)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    a = global_(q, k, v)
    b = global_(q, k, v)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_global_state_only():
    q, k, v = datagen.qkv(1, 4, 5000, 128, 128, 31, 1 / math.sqrt(128), "bf16")
    say("global state only")
    _, S, z = global_(None, k, v)
    _, So, zo, _, _ = oracle.global_(None, f64(k), f64(v))
    check("S", S, So, TOL["bf16"])
    check("z", z[..., None], zo[..., None], TOL["bf16"])


@pytest.mark.parametrize("B,H,N,d,flags", [(2, 4, 3000, 128, 0), (1, 8, 2048, 64, 0), (2, 2, 1500, 128, 3)])
def test_profiled_matches_plain(B, H, N, d, flags):
    """la_causal_fwd_profiled (the entry point the bench times its kernels through) runs the
    same kernels as la_causal_fwd_ex: bit-identical outputs and state, and positive times."""
    m = la()
    q, k, v = datagen.qkv(B, H, N, d, d, 61 + N, 1 / math.sqrt(d), "bf16")
    if flags & 1:  # identity map over positive features
        q, k = q.abs() + 0.05, k.abs() + 0.05
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    say(f"profiled vs plain B={B} H={H} N={N} d={d} flags={flags}")
    outs = []
    for profiled in (False, True):
        out = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        S = torch.full((B, H, d, d), float("nan"), device=DEV)
        z = torch.full((B, H, d), float("nan"), device=DEV)
        if profiled:
            ms = m.la_causal_fwd_profiled(qd, kd, vd, out, None, None, S, z, flags=flags, reps=3)
            assert len(ms) == 3 and all(math.isfinite(t) and t >= 0 for t in ms), ms
            assert ms[2] > 0, ms
        else:
            m.la_causal_fwd_ex(qd, kd, vd, out, None, None, S, z, flags=flags)
        torch.cuda.synchronize()
        outs.append((out.cpu(), S.cpu(), z.cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def test_global_one_segment_per_head():
    """B * H = 256 heads at d = 128: one segment per head, the sums written straight into S, z
    (the path the decode prior of the bench takes); outputs, and the state-only call."""
    assert la().la_segments(1, 16, 16, 777, 128, 128) == 1
    q, k, v = datagen.qkv(16, 16, 777, 128, 128, 51, 1 / math.sqrt(128), "bf16")
    say("global one segment per head B=16 H=16 N=777 d=128")
    o, S, z = global_(q, k, v)
    oo, So, zo, _, _ = oracle.global_(f64(q), f64(k), f64(v))
    check("out", o, oo, TOL["bf16"])
    check("S", S, So, TOL["bf16"])
    check("z", z[..., None], zo[..., None], TOL["bf16"])
    _, S2, z2 = global_(None, k, v)
    assert np.array_equal(S2, S) and np.array_equal(z2, z)


def test_causal_last_row_equals_global():
    q, k, v = datagen.qkv(1, 2, 1500, 64, 64, 41, 1 / 8, "bf16")
    say("causal last row vs global")
    oc, Sc, zc = causal(q, k, v)
    og, Sg, zg = global_(q, k, v)
    check("last row", oc[:, :, -1:], og[:, :, -1:], TOL["bf16"])
    check("state", Sc, Sg, 1e-5)


# ---------------------------------------------------------------- separate initial / final state
@pytest.mark.parametrize("dtype,d,N", [("bf16", 128, 3000), ("bf16", 64, 700), ("f32", 32, 300)])
def test_separate_state(dtype, d, N):
    """la_causal_fwd_state: zero initial state without a buffer; a carried initial state read
    from one buffer and the final state written to another; the initial buffer unchanged."""
    q, k, v = datagen.qkv(2, 3, N, d, d, 51 + d, 1 / math.sqrt(d), dtype)
    n1 = N // 3
    mod = la()
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    say(f"separate state dtype={dtype} d={d} N={N}")
    # first piece from the zero state (nothing to read), final state out
    out_a = torch.empty((2, 3, n1, d), dtype=q.dtype, device=DEV)
    Sa = torch.full((2, 3, d, d), float("nan"), device=DEV)
    za = torch.full((2, 3, d), float("nan"), device=DEV)
    mod.la_causal_fwd_state(qd[:, :, :n1].contiguous(), kd[:, :, :n1].contiguous(),
                            vd[:, :, :n1].contiguous(), out_a, None, None, Sa, za)
    # second piece from that state into fresh buffers
    out_b = torch.empty((2, 3, N - n1, d), dtype=q.dtype, device=DEV)
    Sb = torch.full((2, 3, d, d), float("nan"), device=DEV)
    zb = torch.full((2, 3, d), float("nan"), device=DEV)
    Sa_before = Sa.clone()
    mod.la_causal_fwd_state(qd[:, :, n1:].contiguous(), kd[:, :, n1:].contiguous(),
                            vd[:, :, n1:].contiguous(), out_b, Sa, za, Sb, zb)
    # outputs only (final state not returned)
    out_c = torch.empty_like(out_b)
    mod.la_causal_fwd_state(qd[:, :, n1:].contiguous(), kd[:, :, n1:].contiguous(),
                            vd[:, :, n1:].contiguous(), out_c, Sa, za, None, None)
    torch.cuda.synchronize()
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v))
    _, S1, z1, _, _ = oracle.causal(f64(q[:, :, :n1]), f64(k[:, :, :n1]), f64(v[:, :, :n1]))
    check("first piece out", f64(out_a), oo[:, :, :n1], TOL[dtype])
    check("first piece S", f64(Sa), S1, TOL[dtype])
    check("first piece z", f64(za)[..., None], z1[..., None], TOL[dtype])
    check("second piece out", f64(out_b), oo[:, :, n1:], TOL[dtype])
    check("final S", f64(Sb), So, TOL[dtype])
    check("final z", f64(zb)[..., None], zo[..., None], TOL[dtype])
    assert torch.equal(Sa, Sa_before), "the initial state buffer must not change"
    assert torch.equal(out_b, out_c), "returning the final state must not change the outputs"
