"""Helpers shared by the GPU parity tests: move seeded host inputs to the device, call the
library through its C ABI binding, and bring results back as float64 NumPy arrays."""
from __future__ import annotations

import sys

import numpy as np
import torch

import datagen
from oracle.compare import bounded_row_err, report

DEV = torch.device("cuda:0")


def say(*a):
    """Names the case about to run on the GPU (flushed before the launch)."""
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(t):
    return None if t is None else t.contiguous().to(DEV)


def f64(t):
    return datagen.to_f64(t)


def la():
    import causal_linear_attention_la_amd as m
    return m


def causal(q, k, v, S0=None, z0=None, chunk=0, seg_len=0, want_state=True):
    """Runs la_causal_fwd on host tensors; returns (out, S, z) as float64 arrays."""
    B, H, N, d = q.shape
    dv = v.shape[-1]
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    out = torch.empty((B, H, N, dv), dtype=q.dtype, device=DEV)
    S = z = None
    if want_state or S0 is not None:
        S = to_dev(torch.as_tensor(S0, dtype=torch.float32)) if S0 is not None else \
            torch.zeros((B, H, d, dv), dtype=torch.float32, device=DEV)
        z = to_dev(torch.as_tensor(z0, dtype=torch.float32)) if z0 is not None else \
            torch.zeros((B, H, d), dtype=torch.float32, device=DEV)
    la().la_causal_fwd(qd, kd, vd, out, S, z, chunk=chunk, seg_len=seg_len)
    torch.cuda.synchronize()
    return f64(out), (None if S is None else f64(S)), (None if z is None else f64(z))


def global_(q, k, v, chunk=0):
    B, H, N, d = k.shape
    dv = v.shape[-1]
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    out = None if q is None else torch.empty((B, H, N, dv), dtype=k.dtype, device=DEV)
    S = torch.full((B, H, d, dv), float("nan"), dtype=torch.float32, device=DEV)
    z = torch.full((B, H, d), float("nan"), dtype=torch.float32, device=DEV)
    la().la_global_fwd(qd, kd, vd, out, S, z, chunk=chunk)
    torch.cuda.synchronize()
    return (None if out is None else f64(out)), f64(S), f64(z)


def check(name, got, want, tol):
    r = report(got, want)
    say(f"  {name}: row_max={r['row_max']:.3e} fro={r['fro_rel']:.3e} nonfinite={r['nonfinite']} tol={tol:g}")
    assert r["nonfinite"] == 0, name
    assert r["row_max"] <= tol, (name, r)
    return r


def check_bounded(name, got, want, bound, tol):
    """Forward-error check for sums of signed terms: per row (last axis), the largest error is
    compared with the largest entry of `bound`, the same sum taken over absolute values (the
    scale every rounding error is proportional to). Used where a row's terms may cancel, so
    that the row itself can be far smaller than the terms that make it up."""
    r = bounded_row_err(got, want, bound)
    say(f"  {name}: bounded row_max={r:.3e} nonfinite={int((~np.isfinite(np.asarray(got, dtype=np.float64))).sum())} tol={tol:g}")
    assert r <= tol, (name, r)
    return r
