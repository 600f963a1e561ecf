"""GPU parity of LKV's Soft-TopK (§3.2, App. A.1 forward, App. A.2 backward)
against the fp64 oracle."""
import numpy as np
import pytest
import torch

import future_attention_scoring_kvp_amd as kvp
import oracle
from parity import say, to_dev

pytestmark = pytest.mark.gpu

Y_ATOL = 2e-6      # outputs in (0, 1), computed in fp64 and stored as fp32
LAM_RTOL = 1e-6    # lam stored as fp32


def scores(kind, rows, n, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        v = rng.standard_normal((rows, n)) * 2
    elif kind == "logmass":
        v = np.log(1e-6 + rng.random((rows, n)) ** 6)
    elif kind == "ties":
        v = np.round(rng.standard_normal((rows, n)) * 2) / 2
    elif kind == "equal":
        v = np.full((rows, n), 1.25)
    elif kind == "gap":  # two clusters 1000 apart: exponentials across the gap underflow
        v = rng.standard_normal((rows, n)) + np.where(np.arange(n) % 2 == 0, -500.0, 500.0)
    else:
        raise ValueError(kind)
    return v.astype(np.float32)


def check_fwd(x32, k, tau):
    rows, n = x32.shape
    say(f"[softtopk] rows={rows} n={n} tau={tau}")
    kk = np.broadcast_to(np.asarray(k, np.float32), (rows,)).copy()
    y, lam = kvp.soft_topk(to_dev(x32), to_dev(kk), tau)
    torch.cuda.synchronize()
    ref_y, ref_lam = oracle.soft_topk(x32.astype(np.float64), kk.astype(np.float64), tau)
    y, lam = y.cpu().numpy().astype(np.float64), lam.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(lam - ref_lam) <= LAM_RTOL * np.maximum(1.0, np.abs(ref_lam))), \
        f"lam {lam[:4]} vs {ref_lam[:4]}"
    bad = np.abs(y - ref_y) > Y_ATOL
    assert not bad.any(), f"{int(bad.sum())} outputs off, e.g. {y[bad][:3]} vs {ref_y[bad][:3]}"
    np.testing.assert_allclose(y.sum(1), kk, rtol=0, atol=n * 1e-7 + 1e-6)
    return y, lam


@pytest.mark.parametrize("kind,rows,n,k,tau", [
    ("normal", 4, 100, 10.0, 1.0), ("normal", 3, 777, 123.4, 0.5), ("logmass", 2, 4096, 2048.0, 1.0),
    ("ties", 3, 500, 50.0, 1.0), ("normal", 2, 64, 0.3, 1.0), ("normal", 2, 64, 63.7, 1.0),
    ("normal", 2, 300, 30.0, 0.01), ("normal", 5, 1, 0.5, 1.0), ("normal", 2, 2, 1.0, 1.0),
    ("equal", 2, 300, 100.0, 1.0), ("equal", 2, 300, 150.0, 1.0), ("equal", 2, 300, 250.0, 1.0),
    ("gap", 2, 1000, 500.0, 0.01), ("gap", 2, 1000, 300.0, 0.1), ("gap", 2, 1000, 700.0, 1.0),
    ("normal", 2, 40000, 20000.0, 1.0), ("gap", 2, 40000, 20000.0, 0.01),
])
def test_soft_topk_forward(kind, rows, n, k, tau):
    check_fwd(scores(kind, rows, n, n + rows), k, tau)


def test_per_row_budgets_and_limits():
    x = scores("normal", 6, 200, 3)
    k = np.array([1.0, 2.5, 50.0, 100.0, 199.0, 150.5], np.float32)
    check_fwd(x, k, 1.0)
    # budgets at the ends: nothing kept / everything kept
    y, lam = kvp.soft_topk(to_dev(x[:2]), to_dev(np.array([0.0, 200.0], np.float32)), 1.0)
    torch.cuda.synchronize()
    assert torch.all(y[0] == 0) and torch.all(y[1] == 1)
    assert lam[0].item() == float("inf") and lam[1].item() == float("-inf")


def test_soft_topk_backward():
    rng = np.random.default_rng(5)
    x = scores("normal", 4, 300, 9)
    dy = rng.standard_normal((4, 300)).astype(np.float32)
    k = np.array([10.0, 0.4, 150.0, 299.5], np.float32)
    y, lam = kvp.soft_topk(to_dev(x), to_dev(k), 0.8)
    dx, dk = kvp.soft_topk_backward(to_dev(x), lam, to_dev(dy), 0.8)
    torch.cuda.synchronize()
    ref_dx, ref_dk = oracle.soft_topk_backward(x.astype(np.float64), lam.cpu().numpy().astype(np.float64),
                                               dy.astype(np.float64), 0.8)
    np.testing.assert_allclose(dx.cpu().numpy(), ref_dx, rtol=1e-5, atol=1e-7)
    np.testing.assert_allclose(dk.cpu().numpy(), ref_dk, rtol=1e-5, atol=1e-7)
    # the outputs sum to k whatever x is: a constant upstream gradient gives dx = 0, dk = 1
    dx1, dk1 = kvp.soft_topk_backward(to_dev(x), lam, torch.ones_like(to_dev(dy)), 0.8)
    torch.cuda.synchronize()
    assert dx1.abs().max().item() < 1e-6 and (dk1 - 1).abs().max().item() < 1e-6


def test_full_length_rows():
    """288 rows of 32768 scores (the (layer, KV head) rows of a 36-layer stack),
    half budget, and the same rows with a 2048-token budget."""
    x = scores("logmass", 288, 32768, 1)
    for k in (16384.0, 2048.0):
        check_fwd(x, k, 1.0)
