"""The parity metric (oracle/compare.py) against hand-computed values, and mutated copies of it
against the same pins (CPU only). The real module is never modified."""
import importlib.util
import os

import numpy as np
import pytest

import oracle.compare as compare
from compare_pins import ALL_PINS

SRC = compare.__file__

# (name, text in compare.py, replacement, occurrence: 0 = every occurrence)
MUTANTS = [
    ("mean_for_row_max", "diff = np.abs(a - e).max(axis=-1)", "diff = np.abs(a - e).mean(axis=-1)", 1),
    ("rows_over_axis0", "max(axis=-1)", "max(axis=0)", 0),
    ("diff_without_abs", "diff = np.abs(a - e).max(axis=-1)", "diff = (a - e).max(axis=-1)", 1),
    ("scale_without_abs", "scale = np.abs(e).max(axis=-1)", "scale = e.max(axis=-1)", 1),
    ("scale_from_actual", "scale = np.abs(e).max(axis=-1)", "scale = np.abs(a).max(axis=-1)", 1),
    ("nan_counts_as_zero", "np.where(np.isnan(r), np.inf, r)", "np.where(np.isnan(r), 0.0, r)", 1),
    ("nan_to_num_clips_inf", "np.where(np.isnan(r), np.inf, r)", "np.nan_to_num(r, nan=np.inf)", 1),
    ("mean_over_rows", "np.where(np.isnan(r), np.inf, r).max()", "np.where(np.isnan(r), np.inf, r).mean()", 1),
    ("zero_row_ignored", "np.where(scale > 0, diff / np.where(scale > 0, scale, 1.0), diff)",
     "np.where(scale > 0, diff / np.where(scale > 0, scale, 1.0), 0.0)", 1),
    ("tensor_wide_scale", "scale = np.abs(e).max(axis=-1)", "scale = np.abs(e).max() + 0 * e[..., 0]", 1),
    ("nonfinite_of_expected", "int((~np.isfinite(a)).sum())", "int((~np.isfinite(e)).sum())", 1),
    ("bounded_mean", "err = np.abs(a - e).max(axis=-1)", "err = np.abs(a - e).mean(axis=-1)", 1),
    ("bounded_scale_min", "np.maximum(b.max(axis=-1)", "np.maximum(b.min(axis=-1)", 1),
    ("loose_bf16", '"bf16": 2e-2', '"bf16": 2e-1', 1),
]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_compare_pin(pin):
    pin(compare)


def _mutate(src, old, new, occ):
    assert old in src, old
    if occ == 0:
        return src.replace(old, new)
    parts = src.split(old)
    assert len(parts) > occ
    return old.join(parts[:occ]) + new + old.join(parts[occ:])


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_metric_mutant(tmp_path, name, old, new, occ):
    with open(SRC) as f:
        src = _mutate(f.read(), old, new, occ)
    path = tmp_path / f"compare_{name}.py"
    path.write_text(src)
    spec = importlib.util.spec_from_file_location(f"compare_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches mutant {name}"
