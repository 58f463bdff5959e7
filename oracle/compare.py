"""Error metrics for comparing an implementation's outputs with the oracle's.

TEST INFRASTRUCTURE ONLY.

The pass criterion is the row-wise max-norm relative error: for every output row (one token
of one head, or one key-feature row of a state),

    err_row = max_j |a_j - e_j| / max_j |e_j|

and the check passes when the largest err_row is within tolerance (1e-5 for float32 inputs,
2e-2 for bfloat16 inputs). Element-wise relative error is ill-posed here: values are
zero-mean, so individual outputs sit arbitrarily close to 0 while the row they belong to does
not. A row whose expected values are all exactly 0 is compared in absolute terms. A row with a
non-finite actual value has error +inf (it fails every tolerance).

For sums of signed terms that may cancel (a row far smaller than the terms that make it up),
``bounded_row_err`` divides each row's largest error by the largest entry of the same sum
taken over absolute values -- the scale that floating-point rounding error is proportional to.
"""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-5, "bf16": 2e-2}


def row_rel_err(actual, expected) -> np.ndarray:
    """Per-row max-norm relative error over the last axis (float64)."""
    a = np.asarray(actual, dtype=np.float64)
    e = np.asarray(expected, dtype=np.float64)
    assert a.shape == e.shape, (a.shape, e.shape)
    diff = np.abs(a - e).max(axis=-1)
    scale = np.abs(e).max(axis=-1)
    return np.where(scale > 0, diff / np.where(scale > 0, scale, 1.0), diff)


def _worst(r) -> float:
    """Largest row error; NaN (a non-finite value in the row) counts as +inf."""
    r = np.asarray(r, dtype=np.float64)
    return float(np.where(np.isnan(r), np.inf, r).max()) if r.size else 0.0


def max_row_rel_err(actual, expected) -> float:
    return _worst(row_rel_err(actual, expected))


def bounded_row_err(actual, expected, bound) -> float:
    """Largest over rows of max_j |a_j - e_j| / max_j bound_j (last axis), where ``bound`` holds
    the same sums as ``expected`` taken over absolute values; +inf if any actual value is not
    finite."""
    a, e, b = (np.asarray(x, dtype=np.float64) for x in (actual, expected, bound))
    assert a.shape == e.shape == b.shape, (a.shape, e.shape, b.shape)
    err = np.abs(a - e).max(axis=-1)
    scale = np.maximum(b.max(axis=-1), np.finfo(np.float64).tiny)
    return _worst(err / scale)


def report(actual, expected) -> dict:
    """Row-wise max (the criterion) plus informational figures."""
    a = np.asarray(actual, dtype=np.float64)
    e = np.asarray(expected, dtype=np.float64)
    r = row_rel_err(a, e)
    fro = float(np.linalg.norm(a - e) / max(np.linalg.norm(e), 1e-300))
    return {
        "row_max": _worst(r),
        "row_p99": float(np.percentile(r, 99)) if r.size else 0.0,
        "fro_rel": fro,
        "abs_max": float(np.abs(a - e).max()) if a.size else 0.0,
        "nonfinite": int((~np.isfinite(a)).sum()),
    }
