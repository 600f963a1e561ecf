"""Pins of the oracle's per-head masses and KVpop target scores against
things other than the oracle itself.

The target follows KVpop §3.1 Eq. 2 (future mass with the count
normalisation N_t = max(1, S - (t + w)), App. B.2), Eq. 3 (log(eps + m)
aggregated over the query heads of a group; App. B.1 for the log of the group
mean) and App. B.3 (temporal decay floor((q - t) / n) * log gamma_h).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

from test_oracle_pins import bf16_inputs, widen


def harmonic_table(n):
    h = [Fraction(0)]
    for m in range(1, n + 1):
        h.append(h[-1] + Fraction(1, m))
    return h


def per_head_brute_force(qb, kb, window):
    """Per-query-head column sums of the causal softmax over the rows
    i >= j + window, by scipy on the full matrices."""
    q, k = widen(qb), widen(kb)
    B, Hq, S, D = q.shape
    G = Hq // k.shape[1]
    i_idx, j_idx = np.arange(S)[:, None], np.arange(S)[None, :]
    out = np.zeros((B, Hq, S))
    for b in range(B):
        for g in range(Hq):
            L = np.where(j_idx <= i_idx, (q[b, g] @ k[b, g // G].T) / math.sqrt(D), -np.inf)
            out[b, g] = np.where(i_idx >= j_idx + window, scipy.special.softmax(L, axis=1), 0).sum(0)
    return out


@pytest.mark.parametrize("G,Hkv,S,w", [(1, 1, 40, 0), (4, 2, 33, 5), (2, 3, 50, 49)])
def test_per_head_mass_matrix_brute_force(orc, G, Hkv, S, w):
    rng = np.random.default_rng(S + G)
    qb, kb = bf16_inputs(rng, 1, G * Hkv, Hkv, S, 64, scale=1.3)
    out = orc.future_mass(qb, kb, w, want_per_head=True)
    np.testing.assert_allclose(out["mass_heads"], per_head_brute_force(qb, kb, w), rtol=1e-10,
                               atol=1e-14)
    # the group mass is the sum of its heads' masses
    B, Hq, _ = out["mass_heads"].shape
    np.testing.assert_allclose(out["mass_heads"].reshape(B, Hkv, G, S).sum(2), out["mass"],
                               rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("S,w,normalize", [(64, 8, True), (64, 8, False), (30, 0, True)])
def test_uniform_attention_target_closed_form(orc, S, w, normalize):
    """Q = 0: each head's mass is H_S - H_{t+w}; with N_t the normalised mass
    is (H_S - H_{t+w}) / max(1, S - t - w); every head is the same, so all
    three aggregations give log(eps + m)."""
    rng = np.random.default_rng(7)
    _, kb = bf16_inputs(rng, 1, 2, 2, S, 64)
    qb = np.zeros((1, 6, S, 64), np.uint16)
    heads = orc.future_mass(qb, kb, w, want_per_head=True)["mass_heads"]
    H = harmonic_table(S)
    eps = 1e-3
    exp = []
    for t in range(S):
        m = H[S] - H[t + w] if t + w < S else Fraction(0)
        n_t = max(1, S - (t + w)) if normalize else 1
        exp.append(math.log(eps + float(m / n_t)))
    for agg in (orc.AGG_LOG_MEAN, orc.AGG_MEAN_LOG, orc.AGG_MAX_LOG):
        r = orc.target_scores(heads, w, 2, normalize=normalize, agg=agg, eps=eps)
        np.testing.assert_allclose(r[0, 0], exp, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(r[0, 1], exp, rtol=1e-12, atol=1e-12)


def test_aggregations_order_and_group_sum_path(orc):
    """log is concave: mean of logs <= log of mean <= max of logs, with
    equality only for equal heads; the group-sum input gives the log of the
    mean exactly like the per-head input."""
    rng = np.random.default_rng(11)
    mass = rng.random((2, 8, 100)) ** 3
    r_lm = orc.target_scores(mass, 10, 2, agg=orc.AGG_LOG_MEAN)
    r_ml = orc.target_scores(mass, 10, 2, agg=orc.AGG_MEAN_LOG)
    r_mx = orc.target_scores(mass, 10, 2, agg=orc.AGG_MAX_LOG)
    assert np.all(r_ml <= r_lm + 1e-12) and np.all(r_lm <= r_mx + 1e-12)
    assert np.any(r_ml < r_lm - 1e-6)
    sums = mass.reshape(2, 2, 4, 100).sum(2)
    r_sum = orc.target_scores(sums, 10, 2, per_head=False, group_size=4, agg=orc.AGG_LOG_MEAN)
    np.testing.assert_allclose(r_sum, r_lm, rtol=1e-13, atol=1e-13)
    # one head of the group: all aggregations equal log(eps + m / N_t)
    one = mass[:, :2]
    for agg in (0, 1, 2):
        r = orc.target_scores(one, 10, 2, agg=agg, eps=1e-6)
        n_t = np.maximum(1, 100 - (np.arange(100) + 10))
        np.testing.assert_allclose(r, np.log(1e-6 + one / n_t), rtol=1e-13)


def test_decay_steps(orc):
    """App. B.3: the decay term is zero for q - t < n, log gamma for
    n <= q - t < 2n, ...; tokens after q do not exist (-inf)."""
    S, n, q = 40, 4, 30
    mass = np.full((1, 2, S), 0.25)
    lg = np.array([math.log(0.5), math.log(0.9)])
    base = orc.target_scores(mass, 3, 2, agg=orc.AGG_LOG_MEAN)
    dec = orc.target_scores(mass, 3, 2, agg=orc.AGG_LOG_MEAN, query=q, decay_step=n,
                            log_gamma=lg)
    diff = dec - base
    for t, steps in [(30, 0), (27, 0), (26, 1), (23, 1), (22, 2), (0, 7)]:
        np.testing.assert_allclose(diff[0, :, t], steps * lg, rtol=1e-14, atol=1e-14)
    assert np.all(np.isneginf(dec[:, :, q + 1:]))
    # older tokens decay more: scores of equal masses decrease with age
    assert np.all(np.diff(dec[0, 0, :q + 1]) >= 0)
