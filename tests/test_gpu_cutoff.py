"""GPU parity of the running top-k cutoff (KVpop §3.2, running top-k sparse
attention and its kernel; Appendix I): static ranks and per-query cutoff
ranks, bit-exact against the oracle's Fenwick-tree sweep on the same fp32
scores (widened exactly to fp64), and the last query's retained set against
the one-shot keep-set of kvp_select_topk."""
import numpy as np
import pytest
import torch

import future_attention_scoring_kvp_amd as kvp
import kvp_inputs
import oracle
from parity import say, to_dev

pytestmark = pytest.mark.gpu


def scores(kind, rows, S, seed):
    rng = np.random.default_rng(seed)
    if kind == "ties":      # few distinct values: long runs of equal scores
        v = np.round(rng.standard_normal((rows, S)) * 2) / 4
    elif kind == "logmass":  # negative log-masses, heavy tail
        v = np.log(1e-6 + rng.random((rows, S)) ** 6)
    elif kind == "signed":   # both signs, signed zeros and -inf
        v = rng.standard_normal((rows, S))
        v[:, ::7] = 0.0
        v[:, 3::7] = -0.0
        v[:, 5::11] = -np.inf
    elif kind == "const":    # all equal: the order is the index order
        v = np.full((rows, S), 0.5)
    else:
        raise ValueError(kind)
    return v.astype(np.float32)


def check(score32, window, n_sink, top_k):
    rows, S = score32.shape
    say(f"[cutoff] rows={rows} S={S} w={window} s={n_sink} k={top_k}")
    rank, cut = kvp.running_cutoff(to_dev(score32), window, n_sink, top_k)
    torch.cuda.synchronize()
    ref_rank, ref_cut = oracle.running_cutoff(score32.astype(np.float64)[None], window, n_sink,
                                              top_k)
    got_rank, got_cut = rank.cpu().numpy(), cut.cpu().numpy()
    bad = np.argwhere(got_rank != ref_rank[0])
    assert bad.size == 0, f"rank differs at {bad[:5].tolist()}"
    bad = np.argwhere(got_cut != ref_cut[0])
    assert bad.size == 0, (f"cutoff differs at {bad[:5].tolist()}: "
                           f"{got_cut[tuple(bad[0])]} vs {ref_cut[0][tuple(bad[0])]}")
    return got_rank, got_cut


@pytest.mark.parametrize("kind,rows,S,w,s,k", [
    ("ties", 3, 300, 20, 4, 32), ("logmass", 2, 1000, 64, 4, 100), ("signed", 4, 777, 0, 0, 1),
    ("const", 2, 513, 16, 8, 40), ("ties", 1, 1, 0, 0, 1), ("ties", 2, 5, 0, 0, 5),
    ("logmass", 5, 4097, 128, 4, 512), ("signed", 3, 2000, 50, 3, 1999),
    # long rows past the budget: groups of 64 queries taken one lane per query
    # from a window of ranks below the cutoff, and (small k: windows too
    # shallow at first) groups swept token by token
    ("logmass", 2, 20000, 64, 4, 200), ("ties", 2, 20000, 0, 0, 5000),
    ("signed", 2, 12345, 300, 2, 40),
    # the sort's inverse permutation: four LDS windows exactly, and past them
    # (written directly)
    ("logmass", 1, 32772, 100, 4, 3000), ("ties", 1, 40000, 64, 4, 20000),
])
def test_cutoff_matches_oracle(kind, rows, S, w, s, k):
    check(scores(kind, rows, S, seed=S + k), w, s, k)


@pytest.mark.parametrize("w,s,k", [(10, 4, 0), (10, 4, 10_000), (300, 4, 8), (0, 300, 8),
                                   (1000, 4, 8), (0, 0, 300)])
def test_cutoff_degenerate(w, s, k):
    """k = 0 (cutoff -1), k beyond the eligible count (cutoff S), window or
    sinks covering the sequence (nothing eligible), every token eligible."""
    check(scores("logmass", 2, 300, seed=w + s + k), w, s, k)


def test_last_query_keeps_the_select_topk_set():
    S, w, s, k = 3000, 96, 4, 700
    sc = scores("ties", 4, S, seed=5)
    rank, cut = check(sc, w, s, k)
    keep = kvp.select_topk(to_dev(sc), w, s, k).cpu().numpy()
    q = S - 1
    for r in range(sc.shape[0]):
        t = np.arange(S)
        kept = (t < s) | (t > q - w) | ((rank[r] >= 0) & (rank[r] <= cut[r, q]) & (t <= q - w))
        np.testing.assert_array_equal(np.flatnonzero(kept), keep[r])


def test_cutoff_on_gpu_target_scores_full_length():
    """Full-length rows (32768 keys, window 512, 4 sinks, k = 16384) on target
    scores the GPU computed from a generated layer: masses, KVpop target,
    then the cutoff, compared with the oracle on those same fp32 scores."""
    wl = kvp_inputs.workload(4).with_(layers=1, Hq=8, Hkv=2)
    li = kvp_inputs.make_layer(wl)
    q, k = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, k)
    mh = kvp.future_mass_per_head(q, k, lse, wl.window)
    sc = kvp.target_scores(mh, wl.Hkv, wl.window)
    torch.cuda.synchronize()
    check(sc.reshape(-1, wl.S).cpu().numpy(), wl.window, wl.n_sink, wl.top_k)


def test_cutoff_stack_of_layers_random_rows():
    """Many rows at once (36 layers x 8 KV heads at 32768 keys), random
    continuous scores; every row compared."""
    S = 32768
    sc = scores("logmass", 288, S, seed=9)
    check(sc, 512, 4, 16384)


@pytest.mark.parametrize("n,kind", [(1, "logmass"), (16, "logmass"), (7, "ties")])
def test_static_priority_then_cutoff(n, kind):
    """Static priorities (KVpop §3.2 with App. B.3): every value against the
    oracle's fp64 formula rounded once to fp32, then the running cutoff over
    them bit-exact; with n = 1 the retained set at sampled queries equals a
    direct top-k of the decayed scores r + (q - t) log gamma."""
    rows, S, w, s, k = 6, 3001, 64, 4, 300
    r = scores(kind, rows, S, seed=n)
    lg = np.log(np.array([0.5, 0.7, 0.9, 0.97, 0.999, 1.0], dtype=np.float32)).astype(np.float32)
    say(f"[priority] n={n} {kind}")
    pri = kvp.static_priority(to_dev(r.reshape(1, rows, S)), n, to_dev(lg))
    got = pri.cpu().numpy()[0]
    ref = oracle.static_priority(r.astype(np.float64)[None], n, lg.astype(np.float64))[0]
    ref32 = ref.astype(np.float32)
    both_inf = np.isneginf(got) & np.isneginf(ref32)
    ulp = np.spacing(np.abs(ref32)).astype(np.float64)
    with np.errstate(invalid="ignore"):
        bad = ~both_inf & ~(np.abs(got.astype(np.float64) - ref) <= ulp)
    assert not bad.any(), f"{int(bad.sum())} priorities off by more than one ulp"
    rank, cut = check(got, w, s, k)
    if n == 1:
        for h in range(rows):
            for q in (s + w + k - 1, 1000, S - 1):
                elig = np.arange(s, q - w + 1)
                dec = r[h].astype(np.float64) + (q - np.arange(S)) * float(lg[h])
                order = sorted(elig.tolist(), key=lambda t: (-dec[t], t))[:k]
                kept = elig[rank[h, elig] <= cut[h, q]]
                # ties in the decayed scores may round differently in fp32: compare the sets
                # only where the k-th and (k+1)-th decayed scores are apart
                vk = dec[order[-1]]
                rest = [dec[t] for t in elig.tolist() if t not in set(order)]
                if not rest or vk - max(rest) > 1e-4 * (1 + abs(vk)):
                    assert set(kept.tolist()) == set(order), (h, q)
