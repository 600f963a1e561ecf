"""Pins of the oracle's Soft-TopK (LKV, §3.2 "The Differentiable Soft-TopK
Operator": y_i = f(x_i / tau - lambda) with the Laplace CDF f and the
threshold that makes sum_i y_i = k; App. A.1 closed form, App. A.2
gradients) against things other than the oracle's own arithmetic."""
import math

import numpy as np
import pytest
import scipy.optimize


def laplace_cdf(u):
    return 0.5 * (1.0 + np.sign(u) * (1.0 - np.exp(-np.abs(u))))


def lam_by_root_finding(z, k):
    """Brent's method on the strictly decreasing F(lam) = sum f(z - lam) - k."""
    F = lambda lam: laplace_cdf(z - lam).sum() - k
    lo, hi = z.min() - 50.0, z.max() + 50.0
    return scipy.optimize.brentq(F, lo, hi, xtol=1e-14, rtol=1e-15, maxiter=500)


@pytest.mark.parametrize("n,k,tau,seed", [(10, 3.0, 1.0, 0), (50, 12.5, 0.7, 1), (200, 1.0, 2.0, 2),
                                          (64, 0.3, 1.0, 3), (64, 63.8, 1.0, 4),
                                          (300, 150.0, 0.05, 5)])
def test_threshold_matches_root_finding(orc, n, k, tau, seed):
    x = np.random.default_rng(seed).standard_normal((2, n)) * 3
    y, lam = orc.soft_topk(x, k, tau)
    for r in range(2):
        ref = lam_by_root_finding(x[r] / tau, k)
        assert abs(lam[r] - ref) <= 1e-9 * max(1.0, abs(ref))
        assert abs(y[r].sum() - k) <= 1e-10 * n
        assert np.all((y[r] >= 0) & (y[r] <= 1))  # open interval up to fp64 rounding


def test_two_elements_and_equal_elements_closed_forms(orc):
    # n = 2, k = 1: f(u) + f(-u) = 1, so lam is the midpoint and y1 = f((z1 - z2) / 2)
    y, lam = orc.soft_topk(np.array([[1.7, -0.4]]), 1.0)
    assert abs(lam[0] - 0.65) < 1e-12
    assert abs(y[0, 0] - laplace_cdf(np.array(1.05))) < 1e-12
    # all elements equal: every y_i = k / n
    y, lam = orc.soft_topk(np.full((1, 40), 2.5), 7.0)
    np.testing.assert_allclose(y, 7.0 / 40, rtol=1e-12)


def test_translation_invariance_and_order(orc):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, 80))
    y, lam = orc.soft_topk(x, 20.0, 0.5)
    y2, lam2 = orc.soft_topk(x + 3.25, 20.0, 0.5)
    np.testing.assert_allclose(y2, y, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(lam2, lam + 3.25 / 0.5, rtol=1e-12)
    for r in range(3):
        o = np.argsort(-x[r])
        assert np.all(np.diff(y[r][o]) <= 1e-15)


def test_hard_topk_limit_and_ties(orc):
    x = np.random.default_rng(11).permutation(100).astype(np.float64)[None, :]
    y, _ = orc.soft_topk(x, 10.0, 1e-3)
    hard = (x >= 90).astype(np.float64)
    np.testing.assert_allclose(y, hard, atol=1e-12)
    # equal scores get equal weights
    xt = np.array([[3.0, 1.0, 3.0, 0.0, 1.0, 3.0]])
    yt, _ = orc.soft_topk(xt, 2.0)
    assert yt[0, 0] == yt[0, 2] == yt[0, 5] and yt[0, 1] == yt[0, 4]
    assert abs(yt.sum() - 2.0) < 1e-12


@pytest.mark.parametrize("n,k,tau", [(30, 7.3, 1.0), (60, 0.4, 0.8), (25, 24.7, 1.5)])
def test_backward_matches_finite_differences(orc, n, k, tau):
    rng = np.random.default_rng(n)
    x = rng.standard_normal((1, n))
    g = rng.standard_normal((1, n))
    y, lam = orc.soft_topk(x, k, tau)
    dx, dk = orc.soft_topk_backward(x, lam, g, tau)
    h = 1e-6
    num = np.empty(n)
    for j in range(n):
        xp, xm = x.copy(), x.copy()
        xp[0, j] += h
        xm[0, j] -= h
        num[j] = ((orc.soft_topk(xp, k, tau)[0] - orc.soft_topk(xm, k, tau)[0]) * g).sum() / (2 * h)
    np.testing.assert_allclose(dx[0], num, rtol=1e-5, atol=1e-8)
    numk = ((orc.soft_topk(x, k + h, tau)[0] - orc.soft_topk(x, k - h, tau)[0]) * g).sum() / (2 * h)
    assert abs(dk[0] - numk) <= 1e-5 * max(1.0, abs(numk))
    # the output sum is k for every x, so its gradient along x vanishes
    dx1, dk1 = orc.soft_topk_backward(x, lam, np.ones_like(x), tau)
    np.testing.assert_allclose(dx1, 0.0, atol=1e-12)
    assert abs(dk1[0] - 1.0) < 1e-12
