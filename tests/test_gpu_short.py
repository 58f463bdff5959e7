"""GPU parity of the one-chunk evaluation of short causal sequences (at most 64 tokens, d and
d_v in {16, 32}, chunk left to the library, no decay): every (d, d_v), both dtypes, every flag,
lengths 1, 17 and 64, with no initial state, an initial state passed in place (S, z read and
then overwritten) and an initial state with the final state not requested, each against the
float64 oracle at the dtype's tolerance; and the same call with an explicit chunk (the chunked
kernel) agreeing with it."""
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


def _inputs(flags, B, H, N, d, dv, seed, dtype):
    if flags & IDENT and not flags & UNNORM:
        # identity with a division takes positive features
        q = datagen.positive((B, H, N, d), seed, 1 / math.sqrt(d), dtype)
        k = datagen.positive((B, H, N, d), seed + 1, 1 / math.sqrt(d), dtype)
        v = datagen.normal((B, H, N, dv), seed + 2, 1.0, dtype)
        return q, k, v
    return datagen.qkv(B, H, N, d, dv, seed, 1 / math.sqrt(d), dtype)


def _state(flags, B, H, d, dv, seed, dtype):
    """The state after a 24-token prefix of the same kind of inputs (float32)."""
    q, k, v = _inputs(flags, B, H, 24, d, dv, seed, dtype)
    mode, norm = MODE[flags]
    _, S0, z0, _, _ = oracle.causal(f64(q), f64(k), f64(v), mode=mode, normalize=norm)
    return S0.astype(np.float32), z0.astype(np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,dv", [(16, 16), (16, 32), (32, 16), (32, 32)])
@pytest.mark.parametrize("flags", [0, IDENT, UNNORM, IDENT | UNNORM])
@pytest.mark.parametrize("N", [1, 17, 64])
@pytest.mark.parametrize("state", ["none", "in_place", "no_final"])
def test_short_causal(dtype, d, dv, flags, N, state):
    B, H = 2, 3
    seed = 7000 + 97 * d + 13 * dv + 5 * flags + N
    q, k, v = _inputs(flags, B, H, N, d, dv, seed, dtype)
    mode, norm = MODE[flags]
    S0 = z0 = None
    if state != "none":
        S0, z0 = _state(flags, B, H, d, dv, seed + 50, dtype)
    say(f"short causal dtype={dtype} d={d} dv={dv} flags={flags} N={N} state={state}")
    out = torch.empty((B, H, N, dv), dtype=q.dtype, device=DEV)
    if state == "in_place":
        S, z = torch.from_numpy(S0).to(DEV), torch.from_numpy(z0).to(DEV)
        la().la_causal_fwd_ex(to_dev(q), to_dev(k), to_dev(v), out, S, z, S, z, flags=flags)
    elif state == "no_final":
        S = z = None
        la().la_causal_fwd_ex(to_dev(q), to_dev(k), to_dev(v), out, torch.from_numpy(S0).to(DEV),
                              torch.from_numpy(z0).to(DEV), None, None, flags=flags)
    else:
        S = torch.full((B, H, d, dv), float("nan"), device=DEV)
        z = torch.full((B, H, d), float("nan"), device=DEV)
        la().la_causal_fwd_ex(to_dev(q), to_dev(k), to_dev(v), out, None, None, S, z, flags=flags)
    torch.cuda.synchronize()
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v), S0=S0, z0=z0, mode=mode, normalize=norm)
    if flags == IDENT | UNNORM and dtype == "f32":
        # signed features: a row may cancel far below its terms; bound it by the same sums over
        # absolute values
        ab = [np.abs(f64(x)) for x in (q, k, v)]
        Sa = None if S0 is None else np.abs(S0.astype(np.float64))
        za = None if z0 is None else np.abs(z0.astype(np.float64))
        ob, Sb, zb, _, _ = oracle.causal(*ab, S0=Sa, z0=za, mode=mode, normalize=norm)
        check_bounded("out", f64(out), oo, ob, TOL[dtype])
        if S is not None:
            check_bounded("S", f64(S), So, Sb, TOL[dtype])
        return
    check("out", f64(out), oo, TOL[dtype])
    if S is not None:
        check("S", f64(S), So, TOL[dtype])
        check("z", f64(z)[..., None], zo[..., None], TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_short_matches_chunked(dtype):
    """The one-chunk evaluation and the chunked kernel (explicit chunk 16) agree to rounding."""
    q, k, v = datagen.qkv(2, 4, 64, 16, 16, 7100, 0.25, dtype)
    say(f"short vs chunked dtype={dtype}")
    res = []
    for chunk in (0, 16):
        out = torch.empty((2, 4, 64, 16), dtype=q.dtype, device=DEV)
        S = torch.zeros((2, 4, 16, 16), device=DEV)
        z = torch.zeros((2, 4, 16), device=DEV)
        la().la_causal_fwd(to_dev(q), to_dev(k), to_dev(v), out, S, z, chunk=chunk)
        torch.cuda.synchronize()
        res.append((f64(out), f64(S)))
    check("out", res[0][0], res[1][0], 1e-6 if dtype == "f32" else 1e-2)
    check("S", res[0][1], res[1][1], 1e-6)
