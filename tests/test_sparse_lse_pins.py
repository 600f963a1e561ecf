"""Pins of the oracle's sparse log-normaliser (KVpop §3.2: the running top-k
sparse attention keeps, at query q, the sinks, the protected window and the
top-k eligible tokens under static priorities; its per-query
log-normalisers replace the dense ones in the target)."""
import math

import numpy as np
import pytest
import scipy.special

from test_oracle_pins import bf16_inputs, widen


def running_mask(rank, cutoff, window):
    """keep[i, j] for one (b, KV head): j <= i and (i - j < w or rank_j <= cut_i)."""
    S = rank.shape[0]
    i, j = np.arange(S)[:, None], np.arange(S)[None, :]
    return (j <= i) & (((i - j) < window) | (rank[None, :] <= cutoff[:, None]))


def matrix_sparse_lse(qb, kb, window, rank, cutoff):
    q, k = widen(qb), widen(kb)
    B, Hq, S, D = q.shape
    G = Hq // k.shape[1]
    out = np.empty((B, Hq, S))
    for b in range(B):
        for g in range(Hq):
            h = g // G
            logits = q[b, g] @ k[b, h].T / math.sqrt(D)
            m = running_mask(rank[b, h], cutoff[b, h], window)
            with np.errstate(divide="ignore"):
                out[b, g] = scipy.special.logsumexp(np.where(m, logits, -np.inf), axis=1)
    return out


def priorities(rng, B, Hkv, S):
    return np.round(rng.standard_normal((B, Hkv, S)) * 2) / 4  # many ties


@pytest.mark.parametrize("B,Hq,Hkv,S,w,s,k", [(1, 2, 1, 60, 8, 2, 10), (2, 4, 2, 45, 0, 3, 5),
                                              (1, 4, 1, 70, 5, 0, 0), (1, 2, 2, 40, 4, 4, 200)])
def test_sparse_lse_matrix_brute_force(orc, B, Hq, Hkv, S, w, s, k):
    rng = np.random.default_rng(S + k)
    qb, kb = bf16_inputs(rng, B, Hq, Hkv, S, 64, scale=1.2)
    rank, cut = orc.running_cutoff(priorities(rng, B, Hkv, S), w, s, k)
    got = orc.sparse_lse(qb, kb, w, rank, cut)
    np.testing.assert_allclose(got, matrix_sparse_lse(qb, kb, w, rank, cut), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("S,w,s,k", [(80, 8, 4, 20), (50, 0, 3, 7), (64, 16, 0, 0), (30, 1, 0, 3)])
def test_uniform_attention_counts_kept_keys(orc, S, w, s, k):
    """Q = 0: every logit is 0, so the sparse LSE of row i is ln |K(i)| with
    |K(i)| = |sinks up to i| + |window tokens that are not sinks| +
    min(k, number of eligible tokens s <= t <= i - w)."""
    rng = np.random.default_rng(1)
    _, kb = bf16_inputs(rng, 1, 1, 1, S, 64)
    qb = np.zeros((1, 2, S, 64), np.uint16)
    rank, cut = orc.running_cutoff(priorities(rng, 1, 1, S), w, s, k)
    got = orc.sparse_lse(qb, kb, w, rank, cut)
    for i in range(S):
        sinks = min(s, i + 1)
        win = len([j for j in range(max(0, i - w + 1), i + 1) if j >= s])
        elig = max(0, i - w - s + 1)
        n = sinks + win + min(k, elig)
        exp = math.log(n) if n > 0 else -math.inf
        assert got[0, 0, i] == pytest.approx(exp, abs=1e-12) or (n == 0 and got[0, 0, i] == -math.inf)
        assert got[0, 1, i] == got[0, 0, i]


def test_full_budget_is_dense_and_subset_bound(orc):
    rng = np.random.default_rng(3)
    S, w, s = 90, 6, 2
    qb, kb = bf16_inputs(rng, 1, 4, 2, S, 64, scale=1.3)
    dense = orc.future_mass(qb, kb, w)["lse"]
    rank, cut = orc.running_cutoff(priorities(rng, 1, 2, S), w, s, S)  # k >= every eligible count
    np.testing.assert_allclose(orc.sparse_lse(qb, kb, w, rank, cut), dense, rtol=1e-13, atol=1e-13)
    rank, cut = orc.running_cutoff(priorities(rng, 1, 2, S), w, s, 12)
    sparse = orc.sparse_lse(qb, kb, w, rank, cut)
    assert np.all(sparse <= dense + 1e-12)
    assert np.any(sparse < dense - 1e-3)
