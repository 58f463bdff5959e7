"""float64 CPU oracle for normalized kernelized linear attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may use
this package. It shares no code with the HIP library (``causal_linear_attention_la_amd``) and
neither imports the other; the product path never falls back to it.

Two independent formulations live here:
  * ``oracle.c`` (wrapped below): the token-serial recurrence of the pages, in float64;
  * ``brute.py``: the plain pairwise definition o_i = sum_j w_ij v_j / sum_j w_ij with
    w_ij = phi(q_i) . phi(k_j), computed with NumPy over all pairs (tiny sizes only).
``compare.py`` holds the error metric the parity tests use.

Inputs are float64 NumPy arrays holding exactly the values the GPU saw (bf16/fp32 upcast
exactly); shapes q, k [B,H,N,d], v [B,H,N,dv], S [B,H,d,dv], z [B,H,d].
``mode`` = "elu1" applies phi(x) = ELU(x) + 1; "identity" takes q and k as already mapped
(the convention of the pages' worked examples). ``normalize=False`` returns the numerator
phi(q)^T S itself (the unnormalised form). ``gamma`` (causal and decode) decays the carried
state per head (the retention recurrence). ``rf_map`` gives positive random features.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_DIR = Path(__file__).resolve().parent
_SRC = _DIR / "oracle.c"
_LIB = _DIR / "liboracle.so"
_lib = None

_MODES = {"elu1": 0, "identity": 1}


def build(force: bool = False) -> Path:
    """Compile oracle.c with gcc (float64, no FMA contraction, OpenMP over heads)."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(f".so.tmp{os.getpid()}")
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                        "-fPIC", "-shared", str(_SRC), "-o", str(tmp), "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path):
    lib = ctypes.CDLL(str(path))
    P = ctypes.POINTER(ctypes.c_double)
    L = ctypes.c_long
    lib.oracle_causal.argtypes = [P, P, P, P, P, P, P, P, L, L, L, L, ctypes.c_int, P]
    lib.oracle_global.argtypes = [P, P, P, P, P, P, P, P, L, L, L, L, L, ctypes.c_int]
    lib.oracle_decode.argtypes = [P, P, P, P, P, P, L, L, L, ctypes.c_int, P]
    lib.oracle_causal.restype = None
    lib.oracle_global.restype = None
    lib.oracle_decode.restype = None
    lib.oracle_rf_map.argtypes = [P, P, P, L, L, L]
    lib.oracle_rf_map.restype = None
    lib.oracle_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = _bind(_LIB)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def threads(lib=None) -> int:
    """OpenMP threads the C oracle runs on."""
    return int((lib or _load()).oracle_threads())


def set_threads(n: int) -> int:
    """Sets the OpenMP thread count of later oracle calls from this thread; returns the
    previous count (for timing the oracle single-threaded and on all host cores)."""
    _load()
    gomp = ctypes.CDLL("libgomp.so.1")
    prev = int(gomp.omp_get_max_threads())
    gomp.omp_set_num_threads(int(n))
    return prev


def _mode(mode, normalize):
    return _MODES[mode] | (0 if normalize else 2)


def _gamma(gamma, B, H):
    """Per-head decay [H] (or a scalar) -> one value per (b, h) head, or None."""
    if gamma is None:
        return None
    g = np.broadcast_to(np.asarray(gamma, dtype=np.float64), (H,))
    return np.ascontiguousarray(np.tile(g, B))


def causal(q, k, v, S0=None, z0=None, mode: str = "elu1", normalize: bool = True, gamma=None,
           lib=None):
    """Causal recurrence. Returns (o, S_N, z_N, num, den).

    S0, z0 (optional) are the state before the first token (zeros if omitted). gamma (optional,
    scalar or [H]) is the per-head decay of the carried state."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, H, N, d) and v.shape == (B, H, N, dv)
    S = np.zeros((B, H, d, dv)) if S0 is None else _f64(S0).copy()
    z = np.zeros((B, H, d)) if z0 is None else _f64(z0).copy()
    o = np.empty((B, H, N, dv))
    num = np.empty((B, H, N, dv))
    den = np.empty((B, H, N))
    g = _gamma(gamma, B, H)
    (lib or _load()).oracle_causal(_p(q), _p(k), _p(v), _p(o), _p(num), _p(den), _p(S), _p(z),
                                   B * H, N, d, dv, _mode(mode, normalize), _p(g))
    return o, S, z, num, den


def global_(q, k, v, mode: str = "elu1", normalize: bool = True, lib=None):
    """Global (non-causal) form. Returns (o, S, z, num, den).

    q may hold a different number of rows Nq than k and v (each query row is read against the
    state of all N keys), or be None (state only: o, num, den are None)."""
    k, v = _f64(k), _f64(v)
    B, H, N, d = k.shape
    dv = v.shape[-1]
    assert v.shape == (B, H, N, dv)
    S = np.empty((B, H, d, dv))
    z = np.empty((B, H, d))
    if q is None:
        (lib or _load()).oracle_global(None, _p(k), _p(v), None, None, None, _p(S), _p(z),
                                       B * H, N, 0, d, dv, _mode(mode, normalize))
        return None, S, z, None, None
    q = _f64(q)
    Nq = q.shape[2]
    assert q.shape == (B, H, Nq, d)
    o = np.empty((B, H, Nq, dv))
    num = np.empty((B, H, Nq, dv))
    den = np.empty((B, H, Nq))
    (lib or _load()).oracle_global(_p(q), _p(k), _p(v), _p(o), _p(num), _p(den), _p(S), _p(z),
                                   B * H, N, Nq, d, dv, _mode(mode, normalize))
    return o, S, z, num, den


def decode_step(q, k, v, S, z, mode: str = "elu1", normalize: bool = True, gamma=None,
                lib=None):
    """One recurrent step for every head; q, k [B,H,d] (or [B,H,1,d]), v [B,H,dv] (or
    [B,H,1,dv]). Returns (o [B,H,dv], S', z'); the inputs S, z are not modified. gamma as for
    causal."""
    S = _f64(S).copy()
    z = _f64(z).copy()
    B, H, d, dv = S.shape
    q = _f64(q).reshape(B, H, d)
    k = _f64(k).reshape(B, H, d)
    v = _f64(v).reshape(B, H, dv)
    o = np.empty((B, H, dv))
    g = _gamma(gamma, B, H)
    (lib or _load()).oracle_decode(_p(q), _p(k), _p(v), _p(o), _p(S), _p(z), B * H, d, dv,
                                   _mode(mode, normalize), _p(g))
    return o, S, z


def rf_map(x, W, lib=None):
    """Positive random features of x [..., d] for projections W [m, d]: [..., m]."""
    x = _f64(x)
    W = _f64(W)
    m, d = W.shape
    assert x.shape[-1] == d
    f = np.empty(x.shape[:-1] + (m,))
    (lib or _load()).oracle_rf_map(_p(x), _p(W), _p(f), int(np.prod(x.shape[:-1])), d, m)
    return f
