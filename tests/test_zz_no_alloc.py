"""The allocation-free causal entry point (la_causal_fwd_noalloc: segment states in the
library's static per-device scratch array) against the allocating one (la_causal_fwd_ex),
through the C ABI, on two calls in a row -- the second smaller than the first, so it runs over
what the first left in the array."""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import DEV, check, f64, la, say, to_dev

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _pair(mod, B, H, N, d, seed, seg_len=0, flags=0):
    q, k, v = datagen.qkv(B, H, N, d, d, seed, 1 / math.sqrt(d), "bf16")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    res = []
    for noalloc in (True, False):
        out = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        S = torch.full((B, H, d, d), float("nan"), device=DEV)
        z = torch.full((B, H, d), float("nan"), device=DEV)
        fn = mod.la_causal_fwd_noalloc if noalloc else mod.la_causal_fwd_ex
        fn(qd, kd, vd, out, None, None, S, z, seg_len=seg_len, flags=flags)
        torch.cuda.synchronize()
        res.append((out, S, z))
    for a, b in zip(*res):
        assert torch.equal(_bits(a), _bits(b)), "allocation-free form differs"
    return (q, k, v), res[0]


def test_noalloc_two_calls_then_smaller():
    mod = la()
    say("noalloc: B=2 H=16 N=8192 d=128 (the prefill workload), then B=1 H=4 N=3000 d=64")
    need = mod.la_workspace_bytes(0, 2, 16, 8192, 128, 128)
    assert 0 < need <= 64 << 20
    (q, k, v), (out, S, z) = _pair(mod, 2, 16, 8192, 128, 1003)
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v))
    check("large out", f64(out), oo, 2e-2)
    check("large S", f64(S), So, 2e-2)
    (q, k, v), (out, S, z) = _pair(mod, 1, 4, 3000, 64, 1100, seg_len=256)
    oo, So, zo, _, _ = oracle.causal(f64(q), f64(k), f64(v))
    check("small out", f64(out), oo, 2e-2)
    check("small S", f64(S), So, 2e-2)
    check("small z", f64(z)[..., None], zo[..., None], 2e-2)


def test_noalloc_rejects_oversized_scratch():
    """A split needing more than the 64 MiB array is refused before anything is enqueued."""
    mod = la()
    B, H, N, d = 1, 64, 131072, 128
    assert mod.la_workspace_bytes(0, B, H, N, d, d, 0, 64) > 64 << 20
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device=DEV)
    out = torch.empty_like(q)
    with pytest.raises(mod.LAError) as e:
        mod.la_causal_fwd_noalloc(q, q, q, out, seg_len=64)
    assert e.value.status == mod.LA_ENOSPACE
