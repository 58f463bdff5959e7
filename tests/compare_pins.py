"""Pins of the parity metric (oracle/compare.py) against hand-computed values.

Every GPU parity test passes or fails through these functions, so each is checked here on
small arrays whose errors are worked out by hand (the arithmetic is written next to each
case). ``test_compare.py`` runs the pins on the real module and on mutated copies of it:
each plausible slip (a mean for the max, the wrong axis, a dropped absolute value, NaN read as
0, the all-zero-row branch lost, the scale taken from the actual values) must fail a pin.
"""
from __future__ import annotations

import math

import numpy as np


def _eq(got, want, tol=1e-12):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.allclose(got, want, rtol=tol, atol=tol), (got, want)


def pin_row_error_by_hand(cmp):
    """actual [[3, 4.06], [0, 0]] vs expected [[3, 4], [0, 0]]: row 0 has |diff| max 0.06 over
    max |e| = 4 -> 0.015; row 1 is all zero on both sides -> 0 (absolute branch)."""
    a = [[3.0, 4.06], [0.0, 0.0]]
    e = [[3.0, 4.0], [0.0, 0.0]]
    _eq(cmp.row_rel_err(a, e), [0.015, 0.0])
    _eq(cmp.max_row_rel_err(a, e), 0.015)


def pin_zero_row_is_absolute(cmp):
    """An expected row of exact zeros is compared in absolute terms: actual [0.5, -0.25] against
    [0, 0] -> 0.5 (a relative error would be undefined)."""
    _eq(cmp.row_rel_err([[0.5, -0.25]], [[0.0, 0.0]]), [0.5])
    _eq(cmp.row_rel_err([[1e-3, 2.0]], [[0.0, 2.0]]), [5e-4])


def pin_per_row_not_global(cmp):
    """The scale is each row's own: rows [1.1, 0] vs [1, 0] and [0, 100] vs [0, 100] give row
    errors 0.1 and 0; a tensor-wide scale would give 0.1 / 100 = 1e-3, a mean over rows 0.05."""
    a = [[1.1, 0.0], [0.0, 100.0]]
    e = [[1.0, 0.0], [0.0, 100.0]]
    _eq(cmp.row_rel_err(a, e), [0.1, 0.0])
    _eq(cmp.max_row_rel_err(a, e), 0.1)


def pin_last_axis(cmp):
    """Rows run over the last axis: [[1, 2.2], [1, 2]] vs [[1, 2], [1, 2]] -> [0.1, 0] (columns
    would give [0, 0.1]); a [2, 1, 3] input keeps its leading shape [2, 1]."""
    _eq(cmp.row_rel_err([[1.0, 2.2], [1.0, 2.0]], [[1.0, 2.0], [1.0, 2.0]]), [0.1, 0.0])
    a = np.array([[[1.0, -2.0, 4.4]], [[0.0, 0.0, 3.0]]])
    e = np.array([[[1.0, -2.0, 4.0]], [[0.0, 0.3, 3.0]]])
    # row 0: 0.4 / 4 = 0.1; row 1: 0.3 / 3 = 0.1 ... distinct on purpose below
    e[1, 0, 2] = 6.0   # row 1: max |diff| = 3 (6 vs 3) over max |e| = 6 -> 0.5
    _eq(cmp.row_rel_err(a, e), [[0.1], [0.5]])


def pin_absolute_values(cmp):
    """Both the difference and the scale are absolute values: actual [0.9, 2] vs [1, 2] is off
    by 0.1 below (0.1 / 2 = 0.05, not 0); actual [-4.2, 1] vs [-4, 1] scales by |-4| = 4
    (0.2 / 4 = 0.05, not 0.2 / 1)."""
    _eq(cmp.row_rel_err([[0.9, 2.0]], [[1.0, 2.0]]), [0.05])
    _eq(cmp.row_rel_err([[-4.2, 1.0]], [[-4.0, 1.0]]), [0.05])


def pin_scale_is_expected(cmp):
    """The scale comes from the expected (oracle) row: [3, 4.06] vs [3, 4] is 0.06 / 4 = 0.015
    exactly, not 0.06 / 4.06."""
    _eq(cmp.max_row_rel_err([[3.0, 4.06]], [[3.0, 4.0]]), 0.015, tol=1e-15)


def pin_nonfinite_fails(cmp):
    """A NaN or an infinity in the actual values makes its row's error +inf: the worst row is
    +inf and the report counts the non-finite entries."""
    a = [[math.nan, 1.0], [1.0, 1.0]]
    e = [[1.0, 1.0], [1.0, 1.0]]
    assert cmp.max_row_rel_err(a, e) == math.inf
    r = cmp.report(a, e)
    assert r["row_max"] == math.inf and r["nonfinite"] == 1, r
    assert cmp.max_row_rel_err([[math.inf, 0.0]], [[1.0, 0.0]]) == math.inf
    assert cmp.report([[1.0, -math.inf]], [[1.0, 0.0]])["nonfinite"] == 1


def pin_report_by_hand(cmp):
    """report() on [[3, 4.06], [0, 0]] vs [[3, 4], [0, 0]]: row_max 0.015; Frobenius 0.06 / 5 =
    0.012; max absolute 0.06; 99th percentile of the row errors [0.015, 0] (linear
    interpolation) 0.99 * 0.015; no non-finite value."""
    r = cmp.report([[3.0, 4.06], [0.0, 0.0]], [[3.0, 4.0], [0.0, 0.0]])
    _eq(r["row_max"], 0.015)
    _eq(r["fro_rel"], 0.012)
    _eq(r["abs_max"], 0.06)
    _eq(r["row_p99"], 0.99 * 0.015)
    assert r["nonfinite"] == 0


def pin_bounded_by_hand(cmp):
    """bounded_row_err: rows [1, 2.5] vs [1, 2] with bound [3, 5] -> 0.5 / 5 = 0.1; rows
    [0.01, 0] vs [0, 0] with bound [0.4, 0.2] -> 0.01 / 0.4 = 0.025; worst row 0.1. A NaN in
    the actual values gives +inf."""
    a = [[1.0, 2.5], [0.01, 0.0]]
    e = [[1.0, 2.0], [0.0, 0.0]]
    b = [[3.0, 5.0], [0.4, 0.2]]
    _eq(cmp.bounded_row_err(a, e, b), 0.1)
    _eq(cmp.bounded_row_err(a[1:], e[1:], b[1:]), 0.025)
    _eq(cmp.bounded_row_err([[1.0, 1.9]], [[1.0, 2.0]], [[3.0, 5.0]]), 0.02)
    assert cmp.bounded_row_err([[math.nan, 0.0]], [[1.0, 0.0]], [[1.0, 1.0]]) == math.inf


def pin_tolerances(cmp):
    """The bars: 1e-5 for float32 inputs, 2e-2 for bfloat16 inputs."""
    assert cmp.TOL == {"f32": 1e-5, "bf16": 2e-2}, cmp.TOL


ALL_PINS = [pin_row_error_by_hand, pin_zero_row_is_absolute, pin_per_row_not_global,
            pin_last_axis, pin_absolute_values, pin_scale_is_expected, pin_nonfinite_fails,
            pin_report_by_hand, pin_bounded_by_hand, pin_tolerances]
