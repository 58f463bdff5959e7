"""Plain pairwise definition of normalized kernelized attention (float64, NumPy, tiny sizes).

TEST INFRASTRUCTURE ONLY. This is the definition the linear forms reassociate, written out
over all (query, key) pairs without any state:

    w_ij = phi(q_i) . phi(k_j)
    o_i  = sum_{j in W(i)} w_ij v_j / sum_{j in W(i)} w_ij

with W(i) = {j <= i} for the causal form and all j for the global form
("线性注意力从头到尾讲清楚", section 3, the normalized similarity-weighted average;
"Linear Attention Math", section "Replacing the exponential with a kernel feature map";
"Linear Attention: Accumulating KV in a Fixed-Size State", section "Read the state with a
Query", which expands the state read into these per-token weights).
It costs O(N^2) and is used only to pin the recurrence in ``oracle.c``.
"""
from __future__ import annotations

import numpy as np


def phi(x, mode: str = "elu1"):
    x = np.asarray(x, dtype=np.float64)
    if mode == "identity":
        return x
    return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def weights(q, k, causal: bool, mode: str = "elu1", gamma=None):
    """w[..., i, j] = phi(q_i) . phi(k_j), zeroed for j > i when causal. With a per-head decay
    gamma [H] (causal only), w[..., i, j] is further multiplied by gamma^(i - j): the parallel
    form of the retention recurrence (the decay mask over pairs)."""
    w = np.matmul(phi(q, mode), np.swapaxes(phi(k, mode), -1, -2))
    if causal:
        n = w.shape[-1]
        w = w * np.tril(np.ones((n, n)))
        if gamma is not None:
            H = w.shape[-3]
            g = np.broadcast_to(np.asarray(gamma, dtype=np.float64), (H,))
            lag = np.tril(np.arange(n)[:, None] - np.arange(n)[None, :])   # i - j >= 0
            dmask = np.stack([np.tril(gh ** lag) for gh in g])               # [H, n, n]
            w = w * dmask
    return w


def attend(q, k, v, causal: bool, mode: str = "elu1", gamma=None):
    """Returns (o, num, den) of the pairwise form."""
    w = weights(q, k, causal, mode, gamma)
    num = np.matmul(w, np.asarray(v, dtype=np.float64))
    den = w.sum(axis=-1)
    return num / den[..., None], num, den
