"""Pins of the oracle's static priorities (KVpop §3.2 "Running top-k sparse
attention": the top-k at every query is a running threshold over static
token priorities; App. B.3: the decayed score at query q is
r[t] + floor((q - t) / n) log gamma_h).

The pins do not use the oracle's formula: at every query q the retained set
the running cutoff derives from the static priorities is compared with a
brute-force top-k of the decayed scores r(q) computed from App. B.3 directly.
They must agree exactly for n = 1 and at every q with q mod n = n - 1;
elsewhere they may differ only among tokens whose decayed scores lie within
one decay step |log gamma_h| of the k-th best."""
import math

import numpy as np
import pytest


def decayed(r, q, n, lg):
    t = np.arange(len(r))
    return r + ((q - t) // n) * lg


def brute_topk(v, lo, hi, k):
    """The k best of positions [lo, hi) by value descending, index ascending."""
    idx = list(range(lo, hi))
    idx.sort(key=lambda t: (-v[t], t))
    return set(idx[:k])


def retained(rank, cut, lo, hi):
    return {t for t in range(lo, hi) if rank[t] <= cut}


def scores(rng, S):
    # multiples of 1/8 in a narrow range: exact fp64 arithmetic, many ties
    return np.round(rng.standard_normal(S) * 12) / 8


@pytest.mark.parametrize("S,w,s,k", [(60, 4, 2, 5), (97, 0, 0, 12), (120, 16, 4, 30)])
def test_exact_for_unit_decay_step(orc, S, w, s, k):
    rng = np.random.default_rng(S + k)
    lgs = np.array([math.log(0.5), -0.25, -2.0])   # log 0.5 and two exact values
    r = np.stack([scores(rng, S) for _ in range(3)])[None]
    pri = orc.static_priority(r, 1, lgs)
    rank, cut = orc.running_cutoff(pri, w, s, k)
    for h in range(3):
        for q in range(S):
            hi = q - w + 1
            if hi <= s:
                continue
            ref = brute_topk(decayed(r[0, h], q, 1, lgs[h]), s, hi, k)
            assert retained(rank[0, h], cut[0, h, q], s, hi) == ref, (h, q)


@pytest.mark.parametrize("n", [2, 4, 7])
def test_decay_steps_exact_at_step_ends_and_bounded_elsewhere(orc, n):
    rng = np.random.default_rng(n)
    S, w, s, k = 150, 8, 4, 20
    lg = np.array([-0.5, -0.125])
    r = np.stack([scores(rng, S) for _ in range(2)])[None]
    pri = orc.static_priority(r, n, lg)
    rank, cut = orc.running_cutoff(pri, w, s, k)
    differs = 0
    for h in range(2):
        for q in range(S):
            hi = q - w + 1
            if hi <= s:
                continue
            v = decayed(r[0, h], q, n, lg[h])
            ref = brute_topk(v, s, hi, k)
            got = retained(rank[0, h], cut[0, h, q], s, hi)
            if q % n == n - 1:
                assert got == ref, (h, q)
                continue
            if got != ref:
                differs += 1
                vk = sorted((v[t] for t in ref), reverse=True)[-1]   # k-th best decayed score
                for t in got ^ ref:
                    assert abs(v[t] - vk) <= abs(lg[h]) + 1e-12, (h, q, t)
    assert differs > 0   # the discretization is visible on these inputs


def test_priority_values_and_degenerate_cases(orc):
    r = np.array([[[0.0, 1.0, -np.inf, 2.0, 3.0, 0.5]]])
    pri = orc.static_priority(r, 2, np.array([-1.0]))
    # floor(t / 2) = 0, 0, 1, 1, 2, 2 steps of +1 (log gamma = -1)
    np.testing.assert_array_equal(pri[0, 0], [0.0, 1.0, -np.inf, 3.0, 5.0, 2.5])
    # gamma = 1 (log 0): no decay, the priorities are the scores
    np.testing.assert_array_equal(orc.static_priority(r, 3, np.array([0.0])), r)
