"""Parity helpers shared by the GPU tests: device transfer, tolerances and the
keep-set comparison rule.

Tolerances
  * mass: |gpu - oracle| <= 1e-5 + 2e-3 * |oracle| per key (2e-3 relative /
    1e-5 absolute);
  * LSE: |gpu - oracle| <= 1e-4 (natural log).  The fp32 MFMA accumulation
    of 128 exact bf16 products has an absolute error of order 1e-5 in a logit
    of these inputs, and the LSE of order 1e-5 with it; 1e-4 keeps the induced
    mass error (exp of the LSE error) near 1e-4 relative, well inside the mass
    tolerance;
  * keep-sets: identical whenever the oracle's k-th and (k+1)-th eligible
    masses differ by more than the mass tolerance; otherwise every token
    clearly above the k-th mass must be kept, none clearly below it, and the
    size must match.  Sinks and window are always compared exactly.
"""
import sys

import numpy as np
import torch

MASS_RTOL, MASS_ATOL = 2e-3, 1e-5
LSE_ATOL = 1e-4


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def mass_violations(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    return np.abs(gpu.astype(np.float64) - ref) > MASS_ATOL + MASS_RTOL * np.abs(ref)


def assert_mass(gpu, ref, what=""):
    bad = mass_violations(gpu, ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} mass mismatches, e.g. "
                             + ", ".join(f"{tuple(i)}: gpu {gpu[tuple(i)]:.6g} ref {ref[tuple(i)]:.6g}"
                                         for i in idx))


def assert_lse(gpu, ref, what=""):
    err = np.abs(gpu.astype(np.float64) - ref)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite LSE"
    assert err.max() <= LSE_ATOL, f"{what}: LSE max err {err.max():.3g} at {np.unravel_index(err.argmax(), err.shape)}"


def tol(v):
    return MASS_ATOL + MASS_RTOL * abs(v)


def assert_keep_row(keep, mass, S, w, s, k, exact_ref, what="", tol_fn=None):
    """keep: GPU int32 [n_keep]; mass: oracle fp64 [S] scores; exact_ref:
    oracle keep.  tol_fn(v) is the score tolerance at v (default: the mass
    tolerance)."""
    tol = tol_fn or globals()["tol"]
    keep = np.asarray(keep)
    assert keep.shape == exact_ref.shape, f"{what}: size {keep.shape} vs {exact_ref.shape}"
    if np.array_equal(keep, exact_ref):
        return
    assert np.all(np.diff(keep) > 0), f"{what}: keep-set not strictly ascending"
    ks = set(keep.tolist())
    fixed = set(range(min(s, S))) | set(range(max(0, S - w), S))
    assert fixed <= ks, f"{what}: sink/window token missing"
    e_lo, e_hi = s, S - w
    elig = np.arange(e_lo, e_hi) if e_hi > e_lo else np.arange(0)
    kk = min(k, len(elig))
    order = sorted(elig.tolist(), key=lambda j: (-mass[j], j))
    if kk in (0, len(elig)):
        raise AssertionError(f"{what}: keep-set differs with no selection freedom")
    vk = mass[order[kk - 1]]
    vk1 = mass[order[kk]]
    assert vk - vk1 <= tol(vk), (f"{what}: keep-set differs although the k-th and (k+1)-th masses "
                                 f"are separated ({vk:.6g} vs {vk1:.6g})")
    chosen = ks - fixed
    for j in elig.tolist():
        if mass[j] > vk + tol(vk):
            assert j in chosen, f"{what}: token {j} clearly above the cut is missing"
        if mass[j] < vk - tol(vk):
            assert j not in chosen, f"{what}: token {j} clearly below the cut was kept"
    assert ks - fixed - set(elig.tolist()) == set(), f"{what}: kept a token outside the eligible range"


def assert_keep(keep, mass_ref, w, s, k, exact_ref, what="", tol_fn=None):
    B, H, S = mass_ref.shape
    for b in range(B):
        for h in range(H):
            assert_keep_row(keep[b, h], mass_ref[b, h], S, w, s, k, exact_ref[b, h],
                            f"{what} (b={b}, h={h})", tol_fn)
