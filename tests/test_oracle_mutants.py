"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a private copy of ``oracle/oracle.c`` (a dropped
term, a wrong sign or index, a transposed operand, a skipped normalisation), compiles it to a
temporary library and runs every pin against it: at least one pin must fail. The real oracle
is never modified.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from oracle_pins import ALL_PINS, Orc

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c, replacement, occurrence to replace: 0 = every occurrence)
MUTANTS = [
    ("phi_drops_plus_one", "x > 0.0 ? x + 1.0 : exp(x)", "x > 0.0 ? x : exp(x)", 0),
    ("phi_wrong_sign", "x > 0.0 ? x + 1.0 : exp(x)", "x > 0.0 ? x + 1.0 : exp(-x)", 0),
    ("phi_branch_flipped", "x > 0.0 ? x + 1.0 : exp(x)", "x < 0.0 ? x + 1.0 : exp(x)", 0),
    ("z_counts_tokens", "zh[i] += kf[i];", "zh[i] += 1.0;", 1),
    ("no_normalisation", "o[(h * N + t) * dv + j] = nm[j] / dn;",
     "o[(h * N + t) * dv + j] = nm[j];", 1),
    ("read_transposed_state", "nm[j] += qf[i] * Sh[i * dv + j];",
     "nm[j] += qf[i] * Sh[j * d + i];", 1),
    ("key_off_by_one", "const double *kt = k + (h * N + t) * d;",
     "const double *kt = k + (h * N + (t ? t - 1 : t)) * d;", 1),
    ("value_of_next_token", "const double *vt = v + (h * N + t) * dv;",
     "const double *vt = v + (h * N + (t + 1 < N ? t + 1 : t)) * dv;", 1),
    ("global_reads_key", "qf[i] = phi(qt[i], mode);", "qf[i] = phi(k[(h * N + t) * d + i], mode);", 2),
    ("decode_den_uses_key", "dn += phi(qh[i], mode) * zh[i];", "dn += phi(kh[i], mode) * zh[i];", 1),
    ("decode_read_before_write_scale", "Sh[i * dv + j] += kfi * vh[j];",
     "Sh[i * dv + j] += 0.5 * kfi * vh[j];", 1),
    ("unnormalised_flag_ignored", "if (mode & 2) /* unnormalised form: the numerator is the output */\n                dn = 1.0;",
     "", 1),
    ("global_unnormalised_ignored", "            if (mode & 2)\n                dn = 1.0;", "", 1),
    ("decode_unnormalised_ignored", "        if (mode & 2)\n            dn = 1.0;", "", 1),
    ("rf_drops_half_norm", "exp(dot - 0.5 * sq)", "exp(dot)", 1),
    ("rf_scale_by_m", "1.0 / sqrt((double)m)", "1.0 / (double)m", 1),
    ("rf_transposed_projection", "dot += W[r * d + j] * xi[j];", "dot += W[j * m + r] * xi[j];", 1),
    ("rf_sign_of_projection", "exp(dot - 0.5 * sq)", "exp(-dot - 0.5 * sq)", 1),
    ("decay_after_write", "            if (gamma) {\n                for (long i = 0; i < d * dv; ++i)\n                    Sh[i] *= gamma[h];",
     "            if (0) {\n                for (long i = 0; i < d * dv; ++i)\n                    Sh[i] *= gamma[h];", 1),
    ("decay_skips_key_sum", "                for (long i = 0; i < d; ++i)\n                    zh[i] *= gamma[h];",
     "                for (long i = 0; i < d; ++i)\n                    zh[i] *= 1.0;", 1),
    ("decay_first_head_only", "Sh[i] *= gamma[h];", "Sh[i] *= gamma[0];", 0),
    ("decay_squared", "Sh[i] *= gamma[h];", "Sh[i] *= gamma[h] * gamma[h];", 0),
    ("decode_decay_missing", "        if (gamma) {\n            for (long i = 0; i < d * dv; ++i)",
     "        if (0) {\n            for (long i = 0; i < d * dv; ++i)", 1),
]


def _mutate(src, old, new, occ):
    assert old in src, old
    if occ == 0:
        return src.replace(old, new)
    parts = src.split(old)
    assert len(parts) > occ
    return old.join(parts[:occ]) + new + old.join(parts[occ:])


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, golden, name, old, new, occ):
    with open(SRC) as f:
        src = _mutate(f.read(), old, new, occ)
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O1", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", str(c),
                    "-o", str(so), "-lm"], check=True)
    orc = Orc(oracle._bind(so))
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc, golden)
        except (AssertionError, FloatingPointError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches mutant {name}"
