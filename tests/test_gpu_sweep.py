"""GPU parity over a seeded random sweep of the configuration space: both dtypes, every head
size, d != d_v, ragged lengths (many next to a chunk or segment boundary), explicit chunks and
segment lengths, every flag, a per-head decay and a carried initial state, for the causal form
(and the global form where no decay is asked for), each against the float64 oracle at the
dtype's tolerance. The cases are drawn from a fixed generator, so the list is the same on every
run; each case names itself before it runs."""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import DEV, check, check_bounded, f64, la, say, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
IDENT, UNNORM = 1, 2
MODE = {0: ("elu1", True), IDENT: ("identity", True), UNNORM: ("elu1", False),
        IDENT | UNNORM: ("identity", False)}
DIMS = [16, 32, 64, 128]


def _cases(n=60, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        dtype = ["bf16", "f32"][rng.integers(2)]
        # weighted toward the head sizes of the matrix-core kernels
        d = int(rng.choice(DIMS, p=[0.15, 0.15, 0.3, 0.4]))
        dv = d if rng.random() < 0.8 else int(rng.choice(DIMS))
        chunk = int(rng.choice([0, 0, 0, 16, 32, 64, 128]))
        unit = chunk or 64
        base = int(rng.choice([1, 2, 3, 5, 8, 13, 21, 34]))
        N = max(1, base * unit + int(rng.integers(-2, 3)) if rng.random() < 0.6
                else int(rng.integers(1, 2500)))
        seg = 0 if rng.random() < 0.6 else unit * int(rng.integers(1, 6))
        flags = int(rng.choice([0, 0, IDENT, UNNORM, IDENT | UNNORM]))
        decay = bool(rng.random() < 0.3)
        carry = bool(rng.random() < 0.5)
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        code = la().LA_F32 if dtype == "f32" else la().LA_BF16
        if la().la_segments(0, B, H, N, d, dv, chunk, seg, code) <= 0:
            continue   # a chunk or split the shape does not take
        out.append((len(out), dtype, B, H, N, d, dv, chunk, seg, flags, decay, carry))
    return out


def _inputs(flags, B, H, N, d, dv, seed, dtype):
    # identity with a division takes positive features (denominators are sums of positive terms)
    if flags == IDENT:
        q = datagen.positive((B, H, N, d), seed, 1 / math.sqrt(d), dtype)
        k = datagen.positive((B, H, N, d), seed + 1, 1 / math.sqrt(d), dtype)
        v = datagen.normal((B, H, N, dv), seed + 2, 1.0, dtype)
        return q, k, v
    return datagen.qkv(B, H, N, d, dv, seed, 1 / math.sqrt(d), dtype)


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}")
def test_sweep(case):
    i, dtype, B, H, N, d, dv, chunk, seg, flags, decay, carry = case
    mode, norm = MODE[flags]
    say(f"sweep case {i}: dtype={dtype} B={B} H={H} N={N} d={d} dv={dv} chunk={chunk} "
        f"seg_len={seg} flags={flags} decay={decay} carry={carry}")
    q, k, v = _inputs(flags, B, H, N + 40, d, dv, 4000 + i, dtype)
    gamma = np.linspace(0.0, 1.0, H) if decay and H > 1 else (np.array([0.9]) if decay else None)
    S0 = z0 = None
    if carry:   # the state after a 40-token prefix, as float32
        _, S0, z0, _, _ = oracle.causal(f64(q[:, :, :40]), f64(k[:, :, :40]), f64(v[:, :, :40]),
                                        mode=mode, normalize=norm, gamma=gamma)
        S0, z0 = S0.astype(np.float32), z0.astype(np.float32)
    q, k, v = (x[:, :, 40:].contiguous() for x in (q, k, v))

    out = torch.empty((B, H, N, dv), dtype=q.dtype, device=DEV)
    S = torch.full((B, H, d, dv), float("nan"), device=DEV)
    z = torch.full((B, H, d), float("nan"), device=DEV)
    S0d = None if S0 is None else torch.from_numpy(S0).to(DEV)
    z0d = None if z0 is None else torch.from_numpy(z0).to(DEV)
    if decay:
        g = torch.from_numpy(gamma.astype(np.float32)).to(DEV)
        la().la_causal_fwd_decay(to_dev(q), to_dev(k), to_dev(v), out, g, S0d, z0d, S, z,
                                 chunk=chunk, seg_len=seg, flags=flags)
    else:
        la().la_causal_fwd_ex(to_dev(q), to_dev(k), to_dev(v), out, S0d, z0d, S, z, chunk=chunk,
                              seg_len=seg, flags=flags)
    torch.cuda.synchronize()
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v), S0=S0, z0=z0, mode=mode,
                                     normalize=norm, gamma=gamma)
    if flags == IDENT | UNNORM and dtype == "f32":
        # signed features: a row may cancel far below its terms; bound it by the same sums over
        # absolute values (the scale of float32 rounding error)
        ab = [np.abs(f64(x)) for x in (q, k, v)]
        Sa = None if S0 is None else np.abs(S0.astype(np.float64))
        za = None if z0 is None else np.abs(z0.astype(np.float64))
        ob, Sb, zb, _, _ = oracle.causal(*ab, S0=Sa, z0=za, mode=mode, normalize=norm, gamma=gamma)
        check_bounded("out", f64(out), oo, ob, TOL[dtype])
        check_bounded("S", f64(S), So, Sb, TOL[dtype])
        check_bounded("z", f64(z), zo, zb, TOL[dtype])
    else:
        check("out", f64(out), oo, TOL[dtype])
        check("S", f64(S), So, TOL[dtype])
        check("z", f64(z), zo, TOL[dtype])
    if decay:
        return
    og = torch.empty((B, H, N, dv), dtype=q.dtype, device=DEV)
    Sg = torch.full((B, H, d, dv), float("nan"), device=DEV)
    zg = torch.full((B, H, d), float("nan"), device=DEV)
    la().la_global_fwd_ex(to_dev(q), to_dev(k), to_dev(v), og, Sg, zg, chunk=chunk, flags=flags)
    torch.cuda.synchronize()
    oo, So, zo, _, _ = oracle.global_(f64(q), f64(k), f64(v), mode=mode, normalize=norm)
    if flags == IDENT | UNNORM and dtype == "f32":
        ab = [np.abs(f64(x)) for x in (q, k, v)]
        ob, Sb, zb, _, _ = oracle.global_(*ab, mode=mode, normalize=norm)
        check_bounded("global out", f64(og), oo, ob, TOL[dtype])
        check_bounded("global S", f64(Sg), So, Sb, TOL[dtype])
    else:
        check("global out", f64(og), oo, TOL[dtype])
        check("global S", f64(Sg), So, TOL[dtype])
