"""Pins of the float64 oracle against what the pages and the mathematics fix.

Each ``pin_*`` function takes an oracle handle (``Orc``) and raises AssertionError when the
oracle disagrees with a printed worked example, a closed form, an invariant, the pairwise
brute-force definition or a library-routine special case. ``test_oracle.py`` runs them on
the real oracle; ``test_oracle_mutants.py`` runs them on deliberately broken copies of the
oracle to show that each plausible mistake is caught by at least one pin.
"""
from __future__ import annotations

import math

import numpy as np

import oracle
from oracle import brute

RAW_ONE, RAW_THREE, RAW_ZERO = 0.0, 2.0, -1000.0   # phi(0) = 1, phi(2) = 3, phi(-1000) = 0


class Orc:
    """Binds the oracle's functions to one compiled library (the real one or a mutant)."""

    def __init__(self, lib=None):
        self.lib = lib

    def causal(self, *a, **kw):
        return oracle.causal(*a, lib=self.lib, **kw)

    def global_(self, *a, **kw):
        return oracle.global_(*a, lib=self.lib, **kw)

    def decode_step(self, *a, **kw):
        return oracle.decode_step(*a, lib=self.lib, **kw)

    def rf_map(self, *a, **kw):
        return oracle.rf_map(*a, lib=self.lib, **kw)


def _enc(feat):
    """Raw input whose ELU+1 features are the given 0/1/3 feature values."""
    table = {0: RAW_ZERO, 1: RAW_ONE, 3: RAW_THREE}
    return np.vectorize(lambda x: table[int(x)])(np.asarray(feat, dtype=np.float64))


def _t(x):
    """[N, c] -> [1, 1, N, c]"""
    return np.asarray(x, dtype=np.float64)[None, None]


def _close(a, b, tol=1e-13):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.all(np.isfinite(a)), a
    err = np.abs(a - b).max() if a.size else 0.0
    assert err <= tol * max(1.0, np.abs(b).max()), (a, b, err)


# ---------------------------------------------------------------- feature map: closed form
def pin_phi_closed_form(orc: Orc, golden=None):
    """phi(0)=1, phi(1)=2, phi(2)=3, phi(-1)=e^-1, phi(-1000)=0, phi>0: read off the state
    after one token with v = 1 (S = phi(k) v^T = phi(k))."""
    ks = np.array([0.0, 1.0, 2.0, -1.0, -1000.0, 0.5, -0.5, -20.0])
    want = np.array([1.0, 2.0, 3.0, math.exp(-1.0), 0.0, 1.5, math.exp(-0.5), math.exp(-20.0)])
    d = ks.size
    _, S, z, _, _ = orc.causal(_t(np.zeros((1, d))), _t(ks[None]), _t([[1.0]]))
    _close(S[0, 0, :, 0], want)
    _close(z[0, 0], want)
    assert np.all(S[0, 0, :-4, 0] > 0)


# ------------------------------------------------------------- worked example W1 (page 3)
def pin_two_token_read(orc: Orc, golden):
    g = golden("w1_two_token_read.json")
    k, v, q1 = np.array(g["k"], float), np.array(g["v"], float), np.array(g["q_at_position_1"], float)
    p = g["printed"]
    q = np.stack([q1, q1])
    for mode, enc in (("identity", lambda x: x), ("elu1", _enc)):
        o, S1, z1, _, _ = orc.causal(_t(enc(q[:1])), _t(enc(k[:1])), _t(v[:1]), mode=mode)
        _close(S1[0, 0], p["S_after_token_0"])
        _close(z1[0, 0], p["z_after_token_0"])
        _close(o[0, 0, 0], [g["derived"]["output_at_position_0"]])
        o, S2, z2, num, den = orc.causal(_t(enc(q)), _t(enc(k)), _t(v), mode=mode)
        _close(S2[0, 0], p["S_after_token_1"])
        _close(z2[0, 0], p["z_after_token_1"])
        _close(num[0, 0, 1], [p["numerator"]])
        _close(den[0, 0, 1], p["denominator"])
        _close(o[0, 0, 1], [10.0 / 3.0])
    # the pairwise scores printed on the page, and the same output from them
    w = brute.weights(_t(q), _t(k), causal=True, mode="identity")[0, 0, 1]
    _close(w, p["pairwise_scores"])
    _close((w @ v) / w.sum(), [10.0 / 3.0])


def pin_not_softmax(orc: Orc, golden):
    """Softmax over the same scores (1, 2) gives a different value than the kernel read."""
    g = golden("w1_two_token_read.json")
    k, v, q1 = np.array(g["k"], float), np.array(g["v"], float), np.array(g["q_at_position_1"], float)
    o, *_ = orc.causal(_t(np.stack([q1, q1])), _t(k), _t(v), mode="identity")
    soft = (math.e * 2 + math.e ** 2 * 4) / (math.e + math.e ** 2)
    assert abs(soft - 3.4621) < 1e-4
    assert abs(o[0, 0, 1, 0] - soft) > 0.1
    _close(o[0, 0, 1], [10.0 / 3.0])


# ------------------------------------------------------------- worked example W2 (page 1)
def pin_three_token(orc: Orc, golden):
    g = golden("w2_three_token.json")
    k, v = np.array(g["k"], float), np.array(g["v"], float)
    p, dr = g["printed"], g["derived"]
    for mode, enc in (("identity", lambda x: x), ("elu1", _enc)):
        o, S, z, num, den = orc.causal(_t(enc(k)), _t(enc(k)), _t(v), mode=mode)
        _close(S[0, 0], p["S3"])
        _close(z[0, 0], p["z3"])
        _close(o[0, 0], dr["causal_outputs_with_q_equal_k"])
        _close(num[0, 0, 2], p["reads_unnormalised"]["q=[1,0]"])
        _close(den[0, 0, 2], p["denominator_q2"])
        _close(o[0, 0, 2], p["y2"])
        for qs, key in (([0, 1], "q=[0,1]"), ([1, 1], "q=[1,1]")):
            qq = k.copy()
            qq[2] = qs
            o2, _, _, num2, _ = orc.causal(_t(enc(qq)), _t(enc(k)), _t(v), mode=mode)
            _close(num2[0, 0, 2], p["reads_unnormalised"][key])
            _close(o2[0, 0, 2], dr["normalised_reads"][key])


# ------------------------------------------------------------- worked example W3 (page 4)
def pin_decode_example(orc: Orc, golden):
    g = golden("w3_decode_example.json")
    pk, v, pq = np.array(g["phi_k"], float), np.array(g["v"], float), np.array(g["phi_q"], float)
    p = g["printed"]
    for mode, enc in (("identity", lambda x: x), ("elu1", _enc)):
        S = np.zeros((1, 1, 2, 2))
        z = np.zeros((1, 1, 2))
        for t in range(2):
            o, S, z = orc.decode_step(enc(pq)[None, None], enc(pk[t])[None, None],
                                      v[t][None, None], S, z, mode=mode)
        _close(S[0, 0], p["S"])
        _close(z[0, 0], p["z"])
        _close(o[0, 0], p["output"])
        _close(o[0, 0] * p["denominator"], p["numerator"])


# ------------------------------------------------------------- W4 outer product (page 1)
def pin_outer_product(orc: Orc, golden):
    g = golden("w4_outer_product.json")
    for c in g["cases"]:
        k, v = np.array(c["k"], float), np.array(c["v"], float)
        _, S, z = orc.decode_step(np.ones((1, 1, 2)), k[None, None], v[None, None],
                                  np.zeros((1, 1, 2, 2)), np.zeros((1, 1, 2)), mode="identity")
        _close(S[0, 0], c["printed_kvT"])
        _close(z[0, 0], k)


# ------------------------------------------------------------- W5 duplicates (page 1)
def pin_duplicate_value(orc: Orc, golden):
    g = golden("w5_duplicate_value.json")
    v = np.array(g["v"], float)
    p = g["printed"]
    for mode, raw in (("identity", g["score"]), ("elu1", RAW_ONE)):
        q = np.full((2, 1), raw)
        o, _, _, num, _ = orc.causal(_t(q), _t(q), _t(np.stack([v, v])), mode=mode)
        _close(num[0, 0, 0], p["once_unnormalised"])
        _close(num[0, 0, 1], p["twice_unnormalised"])
        _close(o[0, 0, 0], p["normalised"])
        _close(o[0, 0, 1], p["normalised"])


# ------------------------------------------------------------- W6 global example (page 1)
def pin_global_example(orc: Orc, golden):
    g = golden("w6_global_example.json")
    q, k, v = (np.array(g[x], float) for x in ("q", "k", "v"))
    for mode, enc in (("identity", lambda x: x), ("elu1", _enc)):
        o, S, z, _, _ = orc.global_(_t(enc(q)), _t(enc(k)), _t(v), mode=mode)
        _close(S[0, 0], g["printed_state"]["S"])
        _close(z[0, 0], g["printed_state"]["z"])
        _close(o[0, 0], g["derived"]["global_outputs"])


# ------------------------------------------------------------- pairwise brute force
_SHAPES = [(1, 1, 1, 1, 1), (2, 3, 7, 3, 2), (1, 2, 32, 16, 16), (1, 1, 17, 2, 5),
           (1, 1, 24, 5, 3)]


def _rand(shape, seed, scale=1.0):
    B, H, N, d, dv = shape
    g = np.random.default_rng(seed)
    return (g.standard_normal((B, H, N, d)) * scale, g.standard_normal((B, H, N, d)) * scale,
            g.standard_normal((B, H, N, dv)))


def pin_brute_force(orc: Orc, golden=None):
    """Recurrence == pairwise definition (causal and global, ELU+1 and identity on positive
    features), on tiny random inputs, to 1e-12 row-wise."""
    from oracle.compare import max_row_rel_err
    for i, shp in enumerate(_SHAPES):
        q, k, v = _rand(shp, 100 + i, scale=1.5)
        for mode, (qq, kk) in (("elu1", (q, k)), ("identity", (np.abs(q) + 0.1, np.abs(k) + 0.1))):
            oc, _, _, numc, denc = orc.causal(qq, kk, v, mode=mode)
            ob, numb, denb = brute.attend(qq, kk, v, causal=True, mode=mode)
            assert max_row_rel_err(oc, ob) < 1e-12, (shp, mode)
            assert max_row_rel_err(numc, numb) < 1e-12
            assert max_row_rel_err(denc[..., None], denb[..., None]) < 1e-12
            og, _, _, _, _ = orc.global_(qq, kk, v, mode=mode)
            ob, _, _ = brute.attend(qq, kk, v, causal=False, mode=mode)
            assert max_row_rel_err(og, ob) < 1e-12, (shp, mode)


def pin_global_matmul(orc: Orc, golden=None):
    """Global form == the associativity form with library matmuls:
    S = phi(K)^T V, z = phi(K)^T 1, O = phi(Q) S / phi(Q) z."""
    from oracle.compare import max_row_rel_err
    q, k, v = _rand((2, 2, 40, 6, 4), 7)
    o, S, z, _, _ = orc.global_(q, k, v)
    fq, fk = brute.phi(q), brute.phi(k)
    S2 = np.swapaxes(fk, -1, -2) @ v
    z2 = fk.sum(axis=-2)
    o2 = (fq @ S2) / (fq @ z2[..., None])
    assert max_row_rel_err(S, S2) < 1e-12
    assert max_row_rel_err(z, z2) < 1e-12
    assert max_row_rel_err(o, o2) < 1e-12


# ------------------------------------------------------------- forms against each other
def pin_causal_last_equals_global(orc: Orc, golden=None):
    q, k, v = _rand((2, 3, 19, 4, 6), 11)
    oc, Sc, zc, _, _ = orc.causal(q, k, v)
    og, Sg, zg, _, _ = orc.global_(q, k, v)
    _close(oc[:, :, -1], og[:, :, -1], 1e-12)
    _close(Sc, Sg, 1e-12)
    _close(zc, zg, 1e-12)
    assert np.abs(oc[:, :, 0] - og[:, :, 0]).max() > 1e-3   # earlier rows do differ


def pin_decode_chain_equals_causal(orc: Orc, golden=None):
    q, k, v = _rand((1, 2, 9, 5, 3), 12)
    oc, Sc, zc, _, _ = orc.causal(q, k, v)
    S = np.zeros((1, 2, 5, 3))
    z = np.zeros((1, 2, 5))
    for t in range(9):
        o, S, z = orc.decode_step(q[:, :, t], k[:, :, t], v[:, :, t], S, z)
        _close(o, oc[:, :, t], 1e-12)
    _close(S, Sc, 1e-12)
    _close(z, zc, 1e-12)


def pin_split_invariance(orc: Orc, golden=None):
    """causal over [0, N) == causal over [0, N1) then [N1, N) from the carried state, and
    prefill of N tokens then one decode step == causal over N+1 at position N."""
    q, k, v = _rand((2, 1, 23, 3, 4), 13)
    o, S, z, _, _ = orc.causal(q, k, v)
    n1 = 10
    oa, Sa, za, _, _ = orc.causal(q[:, :, :n1], k[:, :, :n1], v[:, :, :n1])
    ob, Sb, zb, _, _ = orc.causal(q[:, :, n1:], k[:, :, n1:], v[:, :, n1:], S0=Sa, z0=za)
    _close(np.concatenate([oa, ob], axis=2), o, 1e-12)
    _close(Sb, S, 1e-12)
    _close(zb, z, 1e-12)
    op, Sp, zp, _, _ = orc.causal(q[:, :, :-1], k[:, :, :-1], v[:, :, :-1])
    od, Sd, zd = orc.decode_step(q[:, :, -1], k[:, :, -1], v[:, :, -1], Sp, zp)
    _close(od, o[:, :, -1], 1e-12)
    _close(Sd, S, 1e-12)


# ------------------------------------------------------------- normalisation invariants
def pin_invariants(orc: Orc, golden=None):
    q, k, v = _rand((2, 2, 15, 4, 3), 14)
    # one token: the output is that token's value (one rounding of w v / w)
    o1, *_ = orc.causal(q[:, :, :1], k[:, :, :1], v[:, :, :1])
    _close(o1[:, :, 0], v[:, :, 0], 1e-15)
    # constant values -> constant output
    vc = np.broadcast_to(np.array([1.25, -3.0, 0.5]), v.shape).copy()
    oc, *_ = orc.causal(q, k, vc)
    _close(oc, vc, 1e-14)
    # affine in v: o(a v + b) = a o(v) + b
    o, *_ = orc.causal(q, k, v)
    oa, *_ = orc.causal(q, k, 2.5 * v - 0.75)
    _close(oa, 2.5 * o - 0.75, 1e-13)
    # every output lies in the per-column hull of the values it averages
    for t in range(v.shape[2]):
        lo = v[:, :, : t + 1].min(axis=2) - 1e-12
        hi = v[:, :, : t + 1].max(axis=2) + 1e-12
        assert np.all(o[:, :, t] >= lo) and np.all(o[:, :, t] <= hi), t
    # the denominator is the score sum, not the token count
    _, _, _, _, den = orc.causal(q, k, v)
    w = brute.weights(q, k, causal=True)
    _close(den, w.sum(axis=-1), 1e-12)


# ------------------------------------------------------------- unnormalised form (pages 1, 4)
def pin_unnormalised_reads(orc: Orc, golden):
    """normalize=False returns the numerator phi(q)^T S itself: the printed reads of S3, the
    printed numerator of the decode example, and the duplicate-value sums, in all three forms;
    on random inputs the unnormalised output times the normalised form's denominator is the
    normalised output's numerator."""
    g = golden("w7_unnormalised_reads.json")
    se, de = g["state_example"], g["decode_example"]
    k, v = np.array(se["k"], float), np.array(se["v"], float)
    for mode, enc in (("identity", lambda x: x), ("elu1", _enc)):
        for qs, key in (([1, 0], "q=[1,0]"), ([0, 1], "q=[0,1]"), ([1, 1], "q=[1,1]")):
            qq = k.copy()
            qq[2] = qs
            o, _, _, num, _ = orc.causal(_t(enc(qq)), _t(enc(k)), _t(v), mode=mode,
                                         normalize=False)
            _close(o[0, 0, 2], se["printed_reads"][key])
            _close(num[0, 0, 2], se["printed_reads"][key])
            og, *_ = orc.global_(_t(enc(np.array([qs], float))), _t(enc(k)), _t(v), mode=mode,
                                 normalize=False)
            _close(og[0, 0, 0], se["printed_reads"][key])
        pk, dv_, pq = (np.array(de[x], float) for x in ("phi_k", "v", "phi_q"))
        S = np.zeros((1, 1, 2, 2))
        z = np.zeros((1, 1, 2))
        for t in range(2):
            o, S, z = orc.decode_step(enc(pq)[None, None], enc(pk[t])[None, None],
                                      dv_[t][None, None], S, z, mode=mode, normalize=False)
        _close(o[0, 0], de["printed_numerator"])
    w5 = golden("w5_duplicate_value.json")
    vv = np.array(w5["v"], float)
    o, *_ = orc.causal(_t(np.full((2, 1), RAW_ONE)), _t(np.full((2, 1), RAW_ONE)),
                       _t(np.stack([vv, vv])), normalize=False)
    _close(o[0, 0, 0], w5["printed"]["once_unnormalised"])
    _close(o[0, 0, 1], w5["printed"]["twice_unnormalised"])
    q, kk, vr = _rand((1, 2, 13, 4, 3), 15)
    on, _, _, _, den = orc.causal(q, kk, vr)
    ou, Su, zu, _, _ = orc.causal(q, kk, vr, normalize=False)
    _close(ou, on * den[..., None], 1e-13)
    og, Sg, zg, _, _ = orc.global_(q, kk, vr)
    _close(Su, Sg, 1e-12)
    _close(zu, zg, 1e-12)


# ------------------------------------------------------------- positive random features (page 4)
def pin_rf_closed_form(orc: Orc, golden=None):
    """f_r(x) = exp(w_r . x - |x|^2 / 2) / sqrt(m): hand-computed values for an asymmetric W
    (a transposed W or a dropped term changes them), W = 0 gives exp(-|x|^2 / 2) / sqrt(m),
    x = 0 gives 1 / sqrt(m), and every feature is strictly positive."""
    W = np.array([[1.0, 2.0], [0.0, -1.0], [0.5, 0.0]])      # m = 3, d = 2
    x = np.array([[1.0, 0.0], [0.0, 0.5], [-1.0, 1.0]])
    s = 1.0 / math.sqrt(3.0)
    want = np.array([
        [math.exp(1.0 - 0.5), math.exp(0.0 - 0.5), math.exp(0.5 - 0.5)],
        [math.exp(1.0 - 0.125), math.exp(-0.5 - 0.125), math.exp(0.0 - 0.125)],
        [math.exp(1.0 - 1.0), math.exp(-1.0 - 1.0), math.exp(-0.5 - 1.0)],
    ]) * s
    _close(orc.rf_map(x, W), want, 1e-14)
    g = np.random.default_rng(16)
    xr = g.standard_normal((5, 7))
    _close(orc.rf_map(xr, np.zeros((4, 7))),
           np.repeat(np.exp(-0.5 * (xr ** 2).sum(-1))[:, None], 4, axis=1) / 2.0, 1e-14)
    _close(orc.rf_map(np.zeros((2, 7)), g.standard_normal((9, 7))), np.full((2, 9), 1 / 3.0),
           1e-15)
    f = orc.rf_map(3.0 * xr, g.standard_normal((64, 7)))
    assert np.all(f > 0) and np.all(np.isfinite(f))


def pin_rf_unbiased(orc: Orc, golden=None):
    """With standard normal projections, f(q) . f(k) averages to exp(q . k): the estimate over
    2^17 seeded features lies within 5 standard errors of exp(q . k) for several pairs, and
    identity-phi attention over the features of q and k lands near softmax attention over the
    raw scores q . k (the kernel the features estimate)."""
    g = np.random.default_rng(17)
    d, m = 4, 1 << 17
    W = g.standard_normal((m, d))
    q = 0.5 * g.standard_normal((6, d))
    k = 0.5 * g.standard_normal((6, d))
    fq, fk = orc.rf_map(q, W), orc.rf_map(k, W)
    for i in range(6):
        terms = fq[i] * fk[i] * m                      # m per-feature estimates of exp(q.k)
        est, se = terms.mean(), terms.std() / math.sqrt(m)
        exact = math.exp(float(q[i] @ k[i]))
        assert abs(est - exact) <= 5 * se, (i, est, exact, se)
        assert abs(est - exact) <= 0.1 * exact, (i, est, exact)
    v = g.standard_normal((6, 3))
    o, *_ = orc.causal(_t(fq), _t(fk), _t(v), mode="identity")
    sc = np.tril(np.exp(q @ k.T))
    soft = (sc @ v) / sc.sum(-1, keepdims=True)
    _close(o[0, 0], soft, 2e-2)


# ------------------------------------------------------------- decayed recurrence (page 4)
def pin_decay_worked(orc: Orc, golden):
    """Hand-derived three-token example of the decayed recurrence (gamma = 0.5), causal and
    as decode steps, unnormalised with the identity map (the retention form as stated)."""
    g = golden("w8_decay_derived.json")
    k, v, dr = np.array(g["k"], float), np.array(g["v"], float), g["derived"]
    for mode, enc in (("identity", lambda x: x), ("elu1", _enc)):
        o, S, z, _, _ = orc.causal(_t(enc(k)), _t(enc(k)), _t(v), mode=mode, normalize=False,
                                   gamma=g["gamma"])
        _close(S[0, 0], dr["S3"])
        _close(z[0, 0], dr["z3"])
        _close(o[0, 0], dr["causal_outputs_unnormalised_q_equal_k"])
        for qs, key in (([1, 0], "q=[1,0]"), ([0, 1], "q=[0,1]"), ([1, 1], "q=[1,1]")):
            Sd, zd = np.zeros((1, 1, 2, 2)), np.zeros((1, 1, 2))
            for t in range(3):
                qq = np.array(qs if t == 2 else k[t], float)
                od, Sd, zd = orc.decode_step(enc(qq)[None, None], enc(k[t])[None, None],
                                             v[t][None, None], Sd, zd, mode=mode,
                                             normalize=False, gamma=g["gamma"])
                if t < 2:
                    _close(Sd[0, 0], dr[f"S{t + 1}"])
            _close(od[0, 0], dr["reads_unnormalised"][key])


def pin_decay_parallel_form(orc: Orc, golden=None):
    """Recurrence with per-head decay == the parallel form sum_{j<=i} gamma^(i-j) w_ij v_j
    (normalised and not, ELU+1 and identity), with a different gamma per head, including
    gamma = 0 and gamma = 1."""
    from oracle.compare import max_row_rel_err
    gam = np.array([0.9, 0.5, 1.0, 0.0])
    q, k, v = _rand((2, 4, 21, 5, 3), 18, scale=1.2)
    for mode, (qq, kk) in (("elu1", (q, k)), ("identity", (np.abs(q) + 0.1, np.abs(k) + 0.1))):
        for norm in (True, False):
            o, _, _, num, den = orc.causal(qq, kk, v, mode=mode, normalize=norm, gamma=gam)
            ob, numb, denb = brute.attend(qq, kk, v, causal=True, mode=mode, gamma=gam)
            assert max_row_rel_err(num, numb) < 1e-12, (mode, norm)
            assert max_row_rel_err(den[..., None], denb[..., None]) < 1e-12
            assert max_row_rel_err(o, ob if norm else numb) < 1e-12


def pin_decay_special_cases(orc: Orc, golden=None):
    """gamma = 1 is the undecayed form exactly; gamma = 0 keeps only the current token
    (normalised output v_t, unnormalised (phi(q_t) . phi(k_t)) v_t); decode steps chain to
    the causal form, and a carried state splits the sequence, under decay."""
    q, k, v = _rand((2, 3, 17, 4, 3), 19)
    a = orc.causal(q, k, v)
    b = orc.causal(q, k, v, gamma=1.0)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    o0, *_ = orc.causal(q, k, v, gamma=0.0)
    _close(o0, v, 1e-14)
    u0, *_ = orc.causal(q, k, v, normalize=False, gamma=0.0)
    s = (brute.phi(q) * brute.phi(k)).sum(-1)
    _close(u0, s[..., None] * v, 1e-13)
    gam = np.array([0.8, 0.6, 0.95])
    oc, Sc, zc, _, _ = orc.causal(q, k, v, gamma=gam)
    S, z = np.zeros((2, 3, 4, 3)), np.zeros((2, 3, 4))
    for t in range(17):
        od, S, z = orc.decode_step(q[:, :, t], k[:, :, t], v[:, :, t], S, z, gamma=gam)
        _close(od, oc[:, :, t], 1e-12)
    _close(S, Sc, 1e-12)
    _close(z, zc, 1e-12)
    n1 = 6
    oa, Sa, za, _, _ = orc.causal(q[:, :, :n1], k[:, :, :n1], v[:, :, :n1], gamma=gam)
    ob, Sb, zb, _, _ = orc.causal(q[:, :, n1:], k[:, :, n1:], v[:, :, n1:], S0=Sa, z0=za,
                                  gamma=gam)
    _close(np.concatenate([oa, ob], axis=2), oc, 1e-12)
    _close(Sb, Sc, 1e-12)


ALL_PINS = [pin_phi_closed_form, pin_two_token_read, pin_not_softmax, pin_three_token,
            pin_decode_example, pin_outer_product, pin_duplicate_value, pin_global_example,
            pin_brute_force, pin_global_matmul, pin_causal_last_equals_global,
            pin_decode_chain_equals_causal, pin_split_invariance, pin_invariants,
            pin_unnormalised_reads, pin_rf_closed_form, pin_rf_unbiased, pin_decay_worked,
            pin_decay_parallel_form, pin_decay_special_cases]
