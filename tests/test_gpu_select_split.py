"""Keep-sets of rows longer than 32768 scores, which the library splits over
many workgroups with their state in the caller's workspace (KVpop §3 Eq. 1
budget, Eq. 4 eligible set, Fig. 1 sinks and window).  Every result is
compared bit for bit with the oracle's full sort of the same fp32 scores
(ties to the lower index, -0 equal to +0), on score rows with many ties,
signed values, -inf, constant rows and degenerate budgets."""
import numpy as np
import pytest
import torch

import future_attention_scoring_kvp_amd as kvp
import oracle
from parity import say

pytestmark = pytest.mark.gpu


def scores(kind, rows, S, rng):
    if kind == "normal":
        return rng.standard_normal((rows, S)).astype(np.float32)
    if kind == "ties":       # a few hundred distinct values: long runs of ties
        return np.round(rng.standard_normal((rows, S)) * 40).astype(np.float32) / 8
    if kind == "mass":       # positive, heavy-tailed, like future masses
        return (rng.standard_normal((rows, S)) ** 2 * np.exp(rng.standard_normal((rows, S)))
                ).astype(np.float32)
    if kind == "signed":     # log-masses with -inf, and signed zeros
        m = np.log(1e-6 + rng.random((rows, S)) ** 6).astype(np.float32)
        m[:, rng.integers(0, S, S // 50)] = -np.inf
        m[:, rng.integers(0, S, S // 50)] = 0.0
        m[:, rng.integers(0, S, S // 50)] = -0.0
        return m
    if kind == "constant":   # every candidate ties
        return np.full((rows, S), 0.25, np.float32)
    if kind == "two":        # two values: the cut falls inside a huge tie run
        return (rng.random((rows, S)) < 0.3).astype(np.float32)
    raise ValueError(kind)


def check(m, w, s, k, what, ws=None):
    dev = torch.from_numpy(m).cuda()
    keep = kvp.select_topk(dev, w, s, k, workspace=ws).cpu().numpy()
    ref = oracle.select(m.reshape(1, *m.shape).astype(np.float64), w, s, k)[0]
    assert keep.shape == ref.shape, what
    bad = np.nonzero(~np.all(keep == ref, axis=-1))[0]
    assert bad.size == 0, f"{what}: rows {bad[:5].tolist()} differ from the oracle's sort"


@pytest.mark.parametrize("kind", ["normal", "ties", "mass", "signed", "constant", "two"])
@pytest.mark.parametrize("S", [32769, 40001, 131072])
def test_split_rows_exact(kind, S):
    rng = np.random.default_rng(S * 7 + len(kind))
    rows = 3
    m = scores(kind, rows, S, rng)
    say(f"[select split] {kind} S={S}")
    for w, s, k in ((1024, 4, 2048), (512, 4, (S - 516) // 2), (0, 0, 1), (128, 16, S - 145)):
        check(m, w, s, k, f"{kind} S={S} w={w} s={s} k={k}")


@pytest.mark.parametrize("w,s,k", [
    (1024, 4, 0),               # nothing eligible is taken
    (1024, 4, 131072),          # every eligible token is taken
    (1024, 4, 131072 - 1028),   # exactly all eligible
    (131072, 4, 10),            # the window covers the row
    (200000, 0, 10),            # window past the row
    (0, 131072, 10),            # sinks cover the row
    (100, 200000, 5),           # sinks past the row
    (1024, 4, 1),
])
def test_split_degenerate_budgets(w, s, k):
    rng = np.random.default_rng(5)
    m = scores("ties", 2, 131072, rng)
    check(m, w, s, k, f"w={w} s={s} k={k}")


def test_split_config5_shape_and_reused_workspace():
    """Eight rows of 131072 (one layer of 8 KV heads at 128K tokens, k = 2048),
    through one workspace reused by two calls; the second call has fewer
    rows, so the workspace's leftovers from the first must not matter."""
    rng = np.random.default_rng(11)
    S, w, s, k = 131072, 1024, 4, 2048
    need = kvp.select_workspace_bytes(8, S, k)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    m = scores("mass", 8, S, rng)
    check(m, w, s, k, "8 rows", ws)
    check(m[:3] * 0.5, w, s, k, "3 rows after 8", ws)


def test_split_longest_row():
    """One row of 2^22 scores (256 chunks of 16384)."""
    rng = np.random.default_rng(3)
    S = 1 << 22
    m = scores("ties", 1, S, rng)
    say("[select split] S=2^22")
    check(m, 4096, 4, 1 << 20, "S=2^22")
    check(m, 4096, 4, 7, "S=2^22 small k")


def test_split_many_rows_batched_layers():
    """Rows of several batches and heads in one call (batch may stack
    layers), unaligned row starts (S odd)."""
    rng = np.random.default_rng(9)
    S = 33333
    m = scores("normal", 24, S, rng).reshape(3, 8, S)
    dev = torch.from_numpy(m).cuda()
    keep = kvp.select_topk(dev, 300, 4, 1000).cpu().numpy()
    ref = oracle.select(m.reshape(24, 1, S).astype(np.float64), 300, 4, 1000).reshape(3, 8, -1)
    assert np.array_equal(keep, ref)


@pytest.mark.parametrize("seed", range(6))
def test_split_random_shapes(seed):
    """Seeded random rows, lengths, windows, sinks, budgets and score kinds."""
    rng = np.random.default_rng(7700 + seed)
    S = int(rng.integers(32769, 300001))
    rows = int(rng.integers(1, 6))
    kind = ["normal", "ties", "mass", "signed", "constant", "two"][seed]
    w = int(rng.integers(0, S // 4))
    s = int(rng.integers(0, 64))
    k = int(rng.integers(0, S))
    say(f"[select split] random {kind} rows={rows} S={S} w={w} s={s} k={k}")
    check(scores(kind, rows, S, rng), w, s, k, f"random {seed}")
