"""Error metrics for comparing an implementation's outputs with the oracle's.

TEST INFRASTRUCTURE ONLY.

The pass criterion is the row-wise max-norm relative error: for every output row (one token
of one head, or one key-feature row of a state),

    err_row = max_j |a_j - e_j| / max_j |e_j|

and the check passes when the largest err_row is within tolerance (1e-5 for float32 inputs,
2e-2 for bfloat16 inputs). Element-wise relative error is ill-posed here: values are
zero-mean, so individual outputs sit arbitrarily close to 0 while the row they belong to does
not. A row whose expected values are all exactly 0 is compared in absolute terms.
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


def max_row_rel_err(actual, expected) -> float:
    r = row_rel_err(actual, expected)
    return float(np.nan_to_num(r, nan=np.inf).max()) if r.size else 0.0


def report(actual, expected) -> dict:
    """Row-wise max (the criterion) plus informational figures."""
    a = np.asarray(actual, dtype=np.float64)
    e = np.asarray(expected, dtype=np.float64)
    r = row_rel_err(a, e)
    fro = float(np.linalg.norm(a - e) / max(np.linalg.norm(e), 1e-300))
    return {
        "row_max": float(np.nan_to_num(r, nan=np.inf).max()) if r.size else 0.0,
        "row_p99": float(np.percentile(r, 99)) if r.size else 0.0,
        "fro_rel": fro,
        "abs_max": float(np.abs(a - e).max()) if a.size else 0.0,
        "nonfinite": int((~np.isfinite(a)).sum()),
    }
