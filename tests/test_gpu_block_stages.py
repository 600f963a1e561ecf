"""Golden-Eviction block scores (ForesightKV's block-level surrogate: the mean
attention of each query block, pooled over the group, and the future score as
the largest block score of the current and later blocks) on a one-workgroup-
per-CU grid of paired tiles, where one tile of each workgroup sweeps down and
the other up.  Block lengths whose pairs fill whole stages take the kernel
that flushes at stage ends (its sweeps start with a few uncomputed query
blocks, a different number for every block start); the others flush after
any step.  Both are checked against the oracle through the attribution of the
block sums: the scores of blocks t and later, times their rows and heads, add
up to the future mass (KVpop §3.1 Eq. 2, un-normalised as in App. B.1) of the
rows from block t on, which the oracle computes by skipping the earlier rows.
The future scores must be the exact suffix maxima of the block scores."""
import numpy as np
import pytest
import torch

import future_attention_scoring_kvp_amd as kvp
import kvp_inputs
import oracle
from parity import assert_mass, say, to_dev

pytestmark = pytest.mark.gpu

B, HQ, HKV, S, W = 2, 32, 8, 16384, 200
G = HQ // HKV


@pytest.fixture(scope="module")
def layer():
    wl = kvp_inputs.workload(2).with_(B=B, Hq=HQ, Hkv=HKV, S=S, window=W, seed=8080)
    li = kvp_inputs.make_layer(wl)
    q, k = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, k)
    torch.cuda.synchronize()
    return li, q, k, lse


@pytest.mark.parametrize("start,L,per_head", [
    (0, 64, False),       # 8 pairs per block: flush at stage ends
    (32, 64, False),
    (96, 256, False),
    (4064, 2048, False),
    (1024, 256, True),    # per head: 8 pairs per block
    (64, 96, False),      # 12 pairs per block: flush after any step
    (160, 32, True),      # 1 pair per block
])
def test_block_sums_attribute_to_rows(layer, start, L, per_head):
    li, q, k, lse = layer
    n = kvp.block_count(S, start, L)
    say(f"[block stages] start={start} L={L} per_head={per_head}: {n} blocks")
    blk, fut = kvp.block_future_scores(q, k, lse, start, L, window=W, per_head=per_head)
    torch.cuda.synchronize()
    blk, fut = blk.cpu().numpy(), fut.cpu().numpy()
    assert blk.shape == fut.shape == (B, HQ if per_head else HKV, n, S)
    assert np.all(np.isfinite(blk)) and np.all(blk >= 0)
    suffix = np.maximum.accumulate(blk[:, :, ::-1], axis=2)[:, :, ::-1]
    assert np.array_equal(fut, suffix)
    rows = np.array([min(S, start + (t + 1) * L) - (start + t * L) for t in range(n)], np.float64)
    heads = 1 if per_head else G
    b, h = B - 1, HKV - 1
    for t in sorted({0, n // 2, n - 1}):
        r0 = start + t * L
        ref = oracle.future_mass(li.q, li.k, W, b_only=b, h_only=h, row_lo=r0,
                                 want_per_head=per_head)
        tail = (blk[b, :, t:].astype(np.float64) * (rows[t:] * heads)[None, :, None]).sum(axis=1)
        if per_head:
            assert_mass(tail[h * G:(h + 1) * G], ref["mass_heads"][b, h * G:(h + 1) * G],
                        f"start={start} L={L} per head, rows >= {r0}")
        else:
            assert_mass(tail[h], ref["mass"][b, h], f"start={start} L={L}, rows >= {r0}")


@pytest.mark.parametrize("seed", range(4))
def test_random_blocks_on_paired_grids(seed):
    """Seeded random block starts and lengths, windows and group sizes on
    grids of paired tiles (two batches of 8 KV heads at S = 16384, or per
    head): every result checked as above."""
    rng = np.random.default_rng(6600 + seed)
    G_ = int(rng.choice([1, 2, 4]))
    per_head = bool(rng.integers(0, 2))
    w = int(rng.integers(0, 600))
    start = int(rng.integers(0, 200)) * 32
    L = int(rng.choice([32, 64, 96, 128, 160, 256, 512, 1024]))
    wl = kvp_inputs.workload(2).with_(B=2, Hq=8 * G_, Hkv=8, S=S, window=w, seed=6700 + seed)
    li = kvp_inputs.make_layer(wl)
    q, k = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, k)
    n = kvp.block_count(S, start, L)
    say(f"[block stages] random {seed}: G={G_} per_head={per_head} w={w} start={start} L={L} "
        f"({n} blocks)")
    blk, fut = kvp.block_future_scores(q, k, lse, start, L, window=w, per_head=per_head)
    torch.cuda.synchronize()
    blk, fut = blk.cpu().numpy(), fut.cpu().numpy()
    assert np.all(np.isfinite(blk)) and np.all(blk >= 0)
    assert np.array_equal(fut, np.maximum.accumulate(blk[:, :, ::-1], axis=2)[:, :, ::-1])
    rows = np.array([min(S, start + (t + 1) * L) - (start + t * L) for t in range(n)], np.float64)
    heads = 1 if per_head else G_
    b, h = 1, int(rng.integers(0, 8))
    for t in sorted({0, n - 1}):
        r0 = start + t * L
        ref = oracle.future_mass(li.q, li.k, w, b_only=b, h_only=h, row_lo=r0,
                                 want_per_head=per_head)
        tail = (blk[b, :, t:].astype(np.float64) * (rows[t:] * heads)[None, :, None]).sum(axis=1)
        if per_head:
            assert_mass(tail[h * G_:(h + 1) * G_], ref["mass_heads"][b, h * G_:(h + 1) * G_],
                        f"random {seed} per head, rows >= {r0}")
        else:
            assert_mass(tail[h], ref["mass"][b, h], f"random {seed}, rows >= {r0}")
