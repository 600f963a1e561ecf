"""Pins of the oracle's Golden-Eviction block and future scores (ForesightKV,
§3.2 "Golden Eviction": block scores pooled over the rows of a query block
and over the query heads of a GQA group; the appendix's block surrogate is
the mean over the block's queries; the future score is the largest block
score of the current and later blocks) against things other than the
oracle itself."""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

from test_oracle_pins import bf16_inputs, widen


def matrix_block_scores(qb, kb, window, start, L, per_head=False):
    """Matrix form: P = softmax(causal(Q K^T / sqrt d)) by scipy; rows of
    each block averaged by a reshape, heads averaged, suffix max by
    np.maximum.accumulate on the reversed block axis."""
    q, k = widen(qb), widen(kb)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    nb = (S - start + L - 1) // L if S > start else 0
    i_idx, j_idx = np.arange(S)[:, None], np.arange(S)[None, :]
    P = np.empty((B, Hq, S, S))
    for b in range(B):
        for g in range(Hq):
            logits = np.where(j_idx <= i_idx, q[b, g] @ k[b, g // G].T / math.sqrt(D), -np.inf)
            P[b, g] = np.where(i_idx >= j_idx + window, scipy.special.softmax(logits, axis=1), 0.0)
    # pad the rows to whole blocks with zeros and divide by the true row counts
    rows = P[:, :, start:, :]
    pad = nb * L - rows.shape[2]
    rows = np.concatenate([rows, np.zeros((B, Hq, pad, S))], axis=2)
    counts = np.array([min(L, S - start - t * L) for t in range(nb)], dtype=np.float64)
    blk = rows.reshape(B, Hq, nb, L, S).sum(3) / counts[None, None, :, None]
    if not per_head:
        blk = blk.reshape(B, Hkv, G, nb, S).mean(2)
    fut = np.flip(np.maximum.accumulate(np.flip(blk, 2), axis=2), 2)
    return blk, fut


@pytest.mark.parametrize("B,Hq,Hkv,S,D,w,start,L,per_head", [
    (1, 2, 1, 40, 64, 0, 8, 8, False),     # whole blocks
    (1, 4, 2, 45, 64, 0, 5, 12, False),    # ragged last block
    (2, 4, 1, 33, 64, 3, 0, 16, False),    # window, blocks from row 0
    (1, 4, 2, 29, 64, 0, 7, 100, True),    # one block longer than the rest of S
    (1, 2, 2, 20, 64, 0, 20, 4, False),    # no block at all
])
def test_block_scores_matrix_brute_force(orc, B, Hq, Hkv, S, D, w, start, L, per_head):
    rng = np.random.default_rng(S * 7 + L)
    qb, kb = bf16_inputs(rng, B, Hq, Hkv, S, D, scale=1.3)
    out = orc.block_scores(qb, kb, w, start, L, per_head=per_head)
    blk, fut = matrix_block_scores(qb, kb, w, start, L, per_head)
    assert out["block"].shape == blk.shape
    np.testing.assert_allclose(out["block"], blk, rtol=1e-10, atol=1e-15)
    np.testing.assert_allclose(out["future"], fut, rtol=1e-10, atol=1e-15)


def harmonic(n):
    return sum((Fraction(1, m) for m in range(1, n + 1)), Fraction(0))


@pytest.mark.parametrize("S,w,start,L", [(50, 0, 10, 8), (64, 4, 0, 16), (37, 0, 12, 10)])
def test_uniform_attention_closed_form(orc, S, w, start, L):
    """Q = 0: p(i->j) = 1/(i+1) for j <= i, the same for every head, so the
    block score of key j in block t (rows a..e) is
    (H_{e+1} - H_{max(a, j+w)}) / (e - a + 1) (0 if j + w > e), in exact
    rationals; the future score is its suffix maximum over t."""
    rng = np.random.default_rng(3)
    _, kb = bf16_inputs(rng, 1, 2, 2, S, 64)
    qb = np.zeros((1, 4, S, 64), np.uint16)
    out = orc.block_scores(qb, kb, w, start, L)
    nb = orc.block_count(S, start, L)
    H = [Fraction(0)]
    for m in range(1, S + 2):
        H.append(H[-1] + Fraction(1, m))
    exp_blk = np.zeros((nb, S))
    for t in range(nb):
        a, e = start + t * L, min(S, start + (t + 1) * L) - 1
        for j in range(S):
            lo = max(a, j + w)
            exp_blk[t, j] = float((H[e + 1] - H[lo]) / (e - a + 1)) if lo <= e else 0.0
    exp_fut = np.flip(np.maximum.accumulate(np.flip(exp_blk, 0), axis=0), 0)
    for h in range(2):
        np.testing.assert_allclose(out["block"][0, h], exp_blk, rtol=1e-13, atol=1e-16)
        np.testing.assert_allclose(out["future"][0, h], exp_fut, rtol=1e-13, atol=1e-16)


def test_blocks_add_up_to_the_future_mass_of_their_rows(orc):
    """Summed over the blocks (times rows x heads), the block scores give the
    future mass of the rows from block_start on: KVpop's Eq. 2 mass with the
    rows below block_start left out."""
    rng = np.random.default_rng(17)
    S, w, start, L, G = 70, 2, 6, 16, 2
    qb, kb = bf16_inputs(rng, 1, 2 * G, 2, S, 64)
    out = orc.block_scores(qb, kb, w, start, L)
    nb = orc.block_count(S, start, L)
    counts = np.array([min(L, S - start - t * L) for t in range(nb)], dtype=np.float64)
    total = (out["block"] * counts[None, None, :, None]).sum(2) * G
    ref = orc.future_mass(qb, kb, w, row_lo=start)["mass"]
    np.testing.assert_allclose(total, ref, rtol=1e-12, atol=1e-15)


def test_group_mean_of_per_head_scores_and_monotone_future(orc):
    rng = np.random.default_rng(23)
    S, start, L = 60, 4, 8
    qb, kb = bf16_inputs(rng, 1, 4, 1, S, 64)
    grp = orc.block_scores(qb, kb, 0, start, L)
    ph = orc.block_scores(qb, kb, 0, start, L, per_head=True)
    np.testing.assert_allclose(ph["block"].mean(1, keepdims=True), grp["block"], rtol=1e-13,
                               atol=1e-16)
    # the future score never increases with the block index and bounds the block score
    assert np.all(np.diff(grp["future"], axis=2) <= 0)
    assert np.all(grp["future"] >= grp["block"])
    # keys after a block receive nothing from it
    nb = grp["block"].shape[2]
    for t in range(nb):
        e = min(S, start + (t + 1) * L)
        assert np.all(grp["block"][0, 0, t, e:] == 0)
