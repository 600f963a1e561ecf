"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a closed form, an invariant fixed by the
mathematics, a special case that reduces to a library routine, or brute force
on tiny inputs.  The oracle follows KVpop §3.1 Eq. 2 / App. B.1 (future mass),
§3.2 Eq. 8 (LSE reuse), §3 Eq. 1 and Eq. 4 (budget, eligible set) and LKV §3
Eq. 1 (causal scaled softmax).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch


def harmonic(n):
    return sum(Fraction(1, m) for m in range(1, n + 1))


def bf16_inputs(rng, B, Hq, Hkv, S, D, scale=1.0):
    q = torch.from_numpy((rng.standard_normal((B, Hq, S, D)) * scale).astype(np.float32))
    k = torch.from_numpy((rng.standard_normal((B, Hkv, S, D)) * scale).astype(np.float32))
    qb = q.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    kb = k.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return qb, kb


def widen(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def brute_force(qb, kb, window, scale=None):
    """Matrix form: P = softmax(causal(Q K^T * scale)) per query head via
    scipy; mass = column sums over rows i >= j + window, summed over each
    group; LSE = scipy logsumexp of the causal row."""
    q, k = widen(qb), widen(kb)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    i_idx = np.arange(S)[:, None]
    j_idx = np.arange(S)[None, :]
    causal = j_idx <= i_idx
    future = i_idx >= j_idx + window
    lse = np.zeros((B, Hq, S))
    mass = np.zeros((B, Hkv, S))
    for b in range(B):
        for g in range(Hq):
            L = (q[b, g] @ k[b, g // G].T) * scale
            L = np.where(causal, L, -np.inf)
            lse[b, g] = scipy.special.logsumexp(L, axis=1)
            P = scipy.special.softmax(L, axis=1)
            mass[b, g // G] += np.where(future, P, 0.0).sum(axis=0)
    return lse, mass


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("S,w,G", [(256, 16, 1), (64, 0, 2), (100, 7, 4), (33, 40, 1), (50, 49, 3)])
def test_uniform_attention_closed_form(orc, S, w, G):
    """Q = 0: every causal row is uniform over i+1 keys, so LSE_i = ln(i+1)
    and mass[j] = G * sum_{i=j+w}^{S-1} 1/(i+1) = G (H_S - H_{j+w})."""
    D = 64
    rng = np.random.default_rng(S * 31 + w)
    _, kb = bf16_inputs(rng, 1, G, 1, S, D)
    qb = np.zeros((1, G, S, D), np.uint16)
    out = orc.future_mass(qb, kb, w)
    np.testing.assert_allclose(out["lse"][0], np.log(np.arange(1, S + 1))[None, :].repeat(G, 0),
                               rtol=0, atol=1e-13)
    HS = harmonic(S)
    exp = np.array([float(G * (HS - harmonic(j + w))) if j + w < S else 0.0 for j in range(S)])
    np.testing.assert_allclose(out["mass"][0, 0], exp, rtol=1e-13, atol=1e-15)
    # mass is exactly 0 where no future query exists (j >= S - w)
    assert np.all(out["mass"][0, 0, max(0, S - w):] == 0.0)


def test_uniform_attention_total_closed_form(orc):
    """Q = 0, S=256, w=16: total mass = sum_{i>=w} (i-w+1)/(i+1); with w=0 it
    is S (each row sums to one)."""
    S, D = 256, 64
    rng = np.random.default_rng(7)
    _, kb = bf16_inputs(rng, 1, 1, 1, S, D)
    qb = np.zeros((1, 1, S, D), np.uint16)
    tot16 = orc.future_mass(qb, kb, 16)["mass"].sum()
    exp16 = float(sum(Fraction(i - 16 + 1, i + 1) for i in range(16, S)))
    assert abs(tot16 - exp16) < 1e-10
    tot0 = orc.future_mass(qb, kb, 0)["mass"].sum()
    assert abs(tot0 - S) < 1e-10


@pytest.mark.parametrize("S,w,s,k", [(256, 16, 4, 32), (100, 10, 0, 5), (64, 0, 4, 100), (40, 50, 4, 8)])
def test_uniform_attention_keep_set_closed_form(orc, S, w, s, k):
    """Q = 0 mass strictly decreases in j over the eligible range, so the
    keep-set is [0, s + k) together with the window [S - w, S)."""
    D = 64
    rng = np.random.default_rng(3)
    _, kb = bf16_inputs(rng, 1, 1, 1, S, D)
    qb = np.zeros((1, 1, S, D), np.uint16)
    mass = orc.future_mass(qb, kb, w)["mass"]
    keep = orc.select(mass, w, s, k)[0, 0]
    exp = sorted(set(range(min(s, S))) | set(range(s, min(s + k, max(S - w, s))))
                 | set(range(max(0, S - w), S)))
    assert keep.tolist() == exp


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("G,Hkv,S,D,w", [
    (1, 1, 17, 64, 0), (2, 1, 33, 64, 5), (4, 2, 48, 128, 1), (8, 1, 64, 128, 63),
    (1, 3, 40, 64, 40), (2, 2, 29, 128, 33), (4, 1, 64, 64, 16),
])
def test_against_matrix_brute_force(orc, G, Hkv, S, D, w):
    rng = np.random.default_rng(1000 + S * 7 + G)
    qb, kb = bf16_inputs(rng, 2, G * Hkv, Hkv, S, D, scale=1.5)
    out = orc.future_mass(qb, kb, w)
    lse_bf, mass_bf = brute_force(qb, kb, w)
    np.testing.assert_allclose(out["lse"], lse_bf, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["mass"], mass_bf, rtol=1e-11, atol=1e-14)


def test_h2o_special_case(orc):
    """w = 0: the mass is H2O accumulated attention, the column sums of the
    causal softmax over all queries (tutorial page, "H2O: evict by accumulated
    attention"); each column-sum total equals G*S."""
    rng = np.random.default_rng(11)
    qb, kb = bf16_inputs(rng, 1, 4, 1, 64, 64)
    q, k = widen(qb), widen(kb)
    acc = np.zeros(64)
    for g in range(4):
        L = q[0, g] @ k[0, 0].T / 8.0
        L[np.triu_indices(64, 1)] = -np.inf
        acc += torch.softmax(torch.from_numpy(L), dim=1).sum(dim=0).numpy()
    out = orc.future_mass(qb, kb, 0)
    np.testing.assert_allclose(out["mass"][0, 0], acc, rtol=1e-12)
    assert abs(out["mass"].sum() - 4 * 64) < 1e-10


def test_explicit_scale(orc):
    rng = np.random.default_rng(5)
    qb, kb = bf16_inputs(rng, 1, 2, 1, 30, 64)
    out = orc.future_mass(qb, kb, 3, scale=0.3)
    lse_bf, mass_bf = brute_force(qb, kb, 3, scale=0.3)
    np.testing.assert_allclose(out["mass"], mass_bf, rtol=1e-11)
    np.testing.assert_allclose(out["lse"], lse_bf, rtol=1e-12)


# ---------------------------------------------------------------- invariants

def test_invariants(orc):
    B, G, Hkv, S, D, w = 2, 4, 2, 96, 64, 9
    rng = np.random.default_rng(21)
    qb, kb = bf16_inputs(rng, B, G * Hkv, Hkv, S, D, scale=2.0)
    out = orc.future_mass(qb, kb, w, want_rowsum=True, want_winmass=True)
    # every softmax row sums to one
    np.testing.assert_allclose(out["rowsum"], 1.0, rtol=0, atol=1e-12)
    # total mass per KV head = sum over its query heads and rows of (1 - in-window mass)
    outside = (out["rowsum"] - out["winmass"]).reshape(B, Hkv, G, S).sum(axis=(2, 3))
    np.testing.assert_allclose(out["mass"].sum(axis=2), outside, rtol=1e-12)
    # no future query for j >= S - w
    assert np.all(out["mass"][:, :, S - w:] == 0.0)
    # 0 <= mass[j] <= G * (number of rows i >= j + w)
    cnt = np.maximum(S - np.arange(S) - w, 0)
    assert np.all(out["mass"] >= 0)
    assert np.all(out["mass"] <= G * cnt[None, None, :] + 1e-12)
    # max logit <= LSE <= max logit + ln(i + 1)
    q, k = widen(qb), widen(kb)
    for b in range(B):
        for g in range(G * Hkv):
            L = q[b, g] @ k[b, g // G].T / 8.0
            L[np.triu_indices(S, 1)] = -np.inf
            mx = L.max(axis=1)
            assert np.all(mx <= out["lse"][b, g] + 1e-12)
            assert np.all(out["lse"][b, g] <= mx + np.log(np.arange(1, S + 1)) + 1e-12)


def test_group_mapping_permutation(orc):
    """Permuting query heads inside a group leaves the mass unchanged;
    moving a head to another group changes it (query head g uses KV head
    g // G: contiguous groups)."""
    B, G, Hkv, S, D, w = 1, 2, 2, 48, 64, 4
    rng = np.random.default_rng(8)
    qb, kb = bf16_inputs(rng, B, G * Hkv, Hkv, S, D, scale=2.0)
    base = orc.future_mass(qb, kb, w)["mass"]
    within = qb[:, [1, 0, 3, 2]].copy()
    np.testing.assert_allclose(orc.future_mass(within, kb, w)["mass"], base, rtol=1e-13)
    across = qb[:, [0, 2, 1, 3]].copy()
    assert not np.allclose(orc.future_mass(across, kb, w)["mass"], base, rtol=1e-3)


def test_needle(orc):
    """K[j*] = alpha*u and every q_i = u: the needle takes (almost) all of
    every row i >= j*, so mass[j*] -> G*(S - j* - w) and it is kept."""
    S, D, G, w, js = 80, 64, 2, 6, 23
    rng = np.random.default_rng(9)
    u = np.ones(D, np.float32)
    q = np.broadcast_to(u, (1, G, S, D)).astype(np.float32).copy()
    k = rng.standard_normal((1, 1, S, D)).astype(np.float32) * 0.25
    k[0, 0, js] = 8.0 * u
    qb = torch.from_numpy(q).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    kb = torch.from_numpy(k).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mass = orc.future_mass(qb, kb, w)["mass"]
    assert abs(mass[0, 0, js] - G * (S - js - w)) < 1e-9
    keep = orc.select(mass, w, 4, 1)[0, 0]
    assert js in keep.tolist()


def test_row_restriction_and_unit_filter(orc):
    """Restricting to one (b, h) and to rows >= row_lo reproduces the full
    result where it is complete (keys j >= row_lo - w)."""
    B, G, Hkv, S, D, w = 2, 2, 2, 70, 64, 5
    rng = np.random.default_rng(4)
    qb, kb = bf16_inputs(rng, B, G * Hkv, Hkv, S, D)
    full = orc.future_mass(qb, kb, w)
    part = orc.future_mass(qb, kb, w, b_only=1, h_only=0, row_lo=40)
    np.testing.assert_array_equal(part["mass"][1, 0, 35:], full["mass"][1, 0, 35:])
    np.testing.assert_array_equal(part["lse"][1, 0:2, 40:], full["lse"][1, 0:2, 40:])
    assert np.isnan(part["mass"][0]).all() and np.isnan(part["mass"][1, 1]).all()


def test_lse_rows_matches_full(orc):
    rng = np.random.default_rng(12)
    qb, kb = bf16_inputs(rng, 2, 4, 2, 50, 64)
    full = orc.future_mass(qb, kb, 3)["lse"]
    rows = np.array([[0, 0, 0], [1, 3, 49], [0, 2, 17], [1, 1, 33]])
    got = orc.lse_rows(qb, kb, rows)
    np.testing.assert_allclose(got, full[rows[:, 0], rows[:, 1], rows[:, 2]], rtol=1e-14)


def test_thread_count_independent(orc):
    rng = np.random.default_rng(13)
    qb, kb = bf16_inputs(rng, 1, 4, 1, 200, 64)
    a = orc.future_mass(qb, kb, 7, nthreads=1)["mass"]
    b = orc.future_mass(qb, kb, 7, nthreads=8)["mass"]
    np.testing.assert_array_equal(a, b)


def test_f32_inputs_rounded_like_bf16(orc):
    """dtype f32 is rounded to bf16 first: identical to feeding the bf16 bits."""
    rng = np.random.default_rng(14)
    q = rng.standard_normal((1, 2, 40, 64)).astype(np.float32)
    k = rng.standard_normal((1, 1, 40, 64)).astype(np.float32)
    qb = torch.from_numpy(q).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    kb = torch.from_numpy(k).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    a = orc.future_mass(q, k, 4)["mass"]
    b = orc.future_mass(qb, kb, 4)["mass"]
    np.testing.assert_array_equal(a, b)
    c = orc.future_mass(q, k, 4, f32_exact=True)["mass"]
    assert not np.array_equal(a, c)


def test_f32_exact_matrix_brute_force(orc):
    """fp32 inputs used as given (not representable in bf16): LSE and mass
    against the scipy matrix form on the same values widened to fp64."""
    rng = np.random.default_rng(15)
    for (B, Hq, Hkv, S, D, w) in ((1, 2, 1, 40, 64, 4), (2, 4, 2, 33, 128, 0)):
        q = (rng.standard_normal((B, Hq, S, D)) * 1.3).astype(np.float32)
        k = (rng.standard_normal((B, Hkv, S, D)) * 1.3).astype(np.float32)
        out = orc.future_mass(q, k, w, f32_exact=True)
        # brute_force widens bf16 bit patterns; give it the fp32 values directly
        qd, kd = q.astype(np.float64), k.astype(np.float64)
        G = Hq // Hkv
        i_idx, j_idx = np.arange(S)[:, None], np.arange(S)[None, :]
        for b in range(B):
            for g in range(Hq):
                L = np.where(j_idx <= i_idx, (qd[b, g] @ kd[b, g // G].T) / math.sqrt(D), -np.inf)
                np.testing.assert_allclose(out["lse"][b, g], scipy.special.logsumexp(L, axis=1),
                                           rtol=1e-12)
        ref_mass = np.zeros((B, Hkv, S))
        for b in range(B):
            for g in range(Hq):
                L = np.where(j_idx <= i_idx, (qd[b, g] @ kd[b, g // G].T) / math.sqrt(D), -np.inf)
                P = scipy.special.softmax(L, axis=1)
                ref_mass[b, g // G] += np.where(i_idx >= j_idx + w, P, 0.0).sum(axis=0)
        np.testing.assert_allclose(out["mass"], ref_mass, rtol=1e-10, atol=1e-14)


def test_bf16_rounding_matches_torch(orc):
    """The oracle's own round-to-nearest-even agrees with torch's fp32->bf16
    conversion on random values, exact ties and edge values."""
    rng = np.random.default_rng(15)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10,
        # exact ties: low 16 bits == 0x8000, both parities of bit 16
        ((rng.integers(0, 2**15, 2000, dtype=np.uint32) << 17) | 0x8000).view(np.float32),
        ((rng.integers(0, 2**15, 2000, dtype=np.uint32) << 17) | 0x18000).view(np.float32),
        np.array([0.0, -0.0, 1e-40, -1e-40, 3.4e38, -3.4e38, 1.0, -1.0], np.float32),
    ])
    x = x[np.isfinite(x)]
    mine = orc.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)


# ---------------------------------------------------------------- selection

def keep_brute(mass, w, s, k):
    S = mass.shape[0]
    sinks = set(range(min(s, S)))
    window = set(range(max(0, S - w), S))
    elig = [j for j in range(s, S - w)]
    winners = sorted(elig, key=lambda j: (-mass[j], j))[:k]
    return sorted(sinks | window | set(winners))


@pytest.mark.parametrize("S,w,s,k", [
    (256, 16, 4, 32), (100, 0, 0, 10), (100, 0, 4, 1000), (50, 60, 4, 3), (50, 50, 4, 3),
    (50, 46, 4, 3), (30, 5, 40, 2), (1, 0, 0, 1), (1, 1, 1, 1), (0, 3, 4, 5), (300, 7, 4, 0),
])
def test_select_vs_brute_force_with_ties(orc, S, w, s, k):
    rng = np.random.default_rng(S + w + s + k)
    # quantised masses -> many exact ties
    mass = np.round(rng.random((2, 3, S)) * 8) / 8
    keep = orc.select(mass, w, s, k)
    for b in range(2):
        for h in range(3):
            assert keep[b, h].tolist() == keep_brute(mass[b, h], w, s, k)


def test_keep_count_formula(orc):
    for S in range(0, 40):
        for w in (0, 1, 5, 39, 40, 41):
            for s in (0, 1, 4, 45):
                for k in (0, 1, 7, 100):
                    closed = (min(s, S) + max(0, S - max(s, S - w)) + min(k, max(0, S - w - s)))
                    assert orc.keep_count(S, w, s, k) == closed
    assert orc.keep_count(256, 16, 4, 32) == 4 + 16 + 32  # KVpop Eq. 1: B = s + w + k
