"""Pins of the oracle's running top-k cutoff (KVpop §3.2, "Running top-k
sparse attention") against brute force and invariants.  At query q the
eligible tokens are E(q) = {s <= t <= q - w} (Eq. 4); the retained long-range
tokens are the k best of E(q) by static priority, ties to the lower index."""
import numpy as np
import pytest


def brute(score, w, s, k):
    """Direct definition: for every q, order E(q) by (priority desc, index asc)
    and take the k-th; ranks by a Python sort of all tokens >= s."""
    S = len(score)
    order = sorted(range(s, S), key=lambda t: (-score[t], t))
    rank = {t: r for r, t in enumerate(order)}
    ranks = [-1] * min(s, S) + [rank[t] for t in range(s, S)]
    cut = []
    for q in range(S):
        elig = [rank[t] for t in range(s, q - w + 1)]
        if k == 0:
            cut.append(-1)
        elif len(elig) < k:
            cut.append(S)
        else:
            cut.append(sorted(elig)[k - 1])
    return np.array(ranks), np.array(cut)


@pytest.mark.parametrize("S,w,s,k", [(1, 0, 0, 1), (30, 3, 2, 4), (64, 0, 0, 10), (64, 70, 4, 8),
                                     (100, 10, 4, 0), (100, 10, 4, 200), (257, 16, 4, 32)])
def test_cutoff_brute_force_with_ties(orc, S, w, s, k):
    rng = np.random.default_rng(S * 7 + k)
    for trial in range(3):
        score = np.round(rng.standard_normal((2, 2, S)) * 3) / 3   # many exact ties
        if trial == 1:
            score[0, 0] = -np.arange(S)                           # strictly decreasing
        rank, cut = orc.running_cutoff(score, w, s, k)
        for b in range(2):
            for h in range(2):
                r_ref, c_ref = brute(score[b, h], w, s, k)
                assert np.array_equal(rank[b, h], r_ref)
                assert np.array_equal(cut[b, h], c_ref)


def test_cutoff_invariants_and_final_keep_set(orc):
    """Once k tokens are eligible the cutoff never rises; exactly k eligible
    tokens have rank <= cutoff; at the last query the retained set is the
    keep-set of the one-shot selection."""
    rng = np.random.default_rng(3)
    S, w, s, k = 2000, 64, 4, 300
    score = rng.standard_normal((1, 3, S))
    rank, cut = orc.running_cutoff(score, w, s, k)
    for h in range(3):
        c = cut[0, h]
        full = np.arange(S) - w - s + 1 >= k   # |E(q)| >= k
        assert np.all(c[~full] == S)
        assert np.all(np.diff(c[full]) <= 0)
        for q in (w + s + k - 1, 1000, S - 1):
            elig = np.arange(s, q - w + 1)
            assert np.sum(rank[0, h, elig] <= c[q]) == k
        kept = sorted(set(range(s)) | set(range(S - w, S)) |
                      {t for t in range(s, S - w) if rank[0, h, t] <= c[S - 1]})
        assert kept == orc.select(score[:, h:h + 1], w, s, k)[0, 0].tolist()


def test_decreasing_priority_closed_form(orc):
    """Priorities that decrease with the index rank tokens in index order, so
    the k best eligible tokens are always the k oldest: cutoff = k - 1."""
    S, w, s, k = 500, 20, 4, 50
    score = -np.arange(S, dtype=np.float64)[None, None]
    rank, cut = orc.running_cutoff(score, w, s, k)
    assert np.array_equal(rank[0, 0, s:], np.arange(S - s))
    first = s + w + k - 1   # query at which k tokens are eligible
    assert np.all(cut[0, 0, :first] == S) and np.all(cut[0, 0, first:] == k - 1)
