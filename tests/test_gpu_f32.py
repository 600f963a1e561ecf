"""fp32 inputs are used as given: the LSE, the future masses (group and per
head), the Golden-Eviction scores and the sparse LSE computed in fp32 on the
vector ALUs, against the oracle in fp64 on the same fp32 values (no bf16
rounding anywhere), at the mass tolerance and the LSE tolerance."""
import numpy as np
import pytest
import torch

import future_attention_scoring_kvp_amd as kvp
import kvp_inputs
import oracle
from parity import LSE_ATOL, assert_lse, assert_mass, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,Hq,Hkv,S,D,w,s,k", [
    (1, 1, 1, 256, 64, 16, 4, 32),        # the tiny workload's shape
    (2, 8, 2, 1500, 128, 40, 4, 300),     # groups of 4, ragged last tiles
    (1, 3, 3, 97, 64, 0, 0, 10),          # one head per group, window 0
])
def test_f32_path_against_exact_oracle(B, Hq, Hkv, S, D, w, s, k):
    wl = kvp_inputs.workload(1).with_(B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, window=w, n_sink=s,
                                      top_k=k, seed=4242 + S)
    li = kvp_inputs.make_layer(wl)
    assert li.q.dtype == np.float32
    say(f"[f32] B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} w={w} s={s} k={k}")
    q, kk = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, kk)
    mass = kvp.future_mass(q, kk, lse, w)
    ph = kvp.future_mass_per_head(q, kk, lse, w)
    blk, fut = kvp.block_future_scores(q, kk, lse, 32, 64, window=w)
    rng = np.random.default_rng(S)
    pri = (np.round(rng.standard_normal((B, Hkv, S)) * 3) / 4).astype(np.float32)
    rank, cut = kvp.running_cutoff(to_dev(pri), w, s, k)
    sp = kvp.lse_sparse(q, kk, rank, cut, w)
    torch.cuda.synchronize()

    ref = oracle.future_mass(li.q, li.k, w, want_per_head=True, f32_exact=True)
    assert_lse(lse.cpu().numpy(), ref["lse"], "f32 lse")
    assert_mass(mass.cpu().numpy(), ref["mass"], "f32 mass")
    assert_mass(ph.cpu().numpy(), ref["mass_heads"], "f32 per-head mass")
    # fp32 arithmetic: far inside the tolerances
    assert np.abs(lse.cpu().numpy() - ref["lse"]).max() <= 1e-5
    rb = oracle.block_scores(li.q, li.k, w, 32, 64, f32_exact=True)
    assert_mass(blk.cpu().numpy(), rb["block"], "f32 block scores")
    assert_mass(fut.cpu().numpy(), rb["future"], "f32 future scores")
    r_rank, r_cut = oracle.running_cutoff(pri.astype(np.float64), w, s, k)
    r_sp = oracle.sparse_lse(li.q, li.k, w, r_rank, r_cut, f32_exact=True)
    got = sp.cpu().numpy().astype(np.float64)
    finite = np.isfinite(r_sp)
    assert np.array_equal(finite, np.isfinite(got))
    if finite.any():
        assert np.abs(got[finite] - r_sp[finite]).max() <= LSE_ATOL


def test_f32_differs_from_rounding_its_inputs():
    """The fp32 path does not round its inputs: on the tiny workload the
    oracle's bf16-rounded result is farther from the GPU than the exact one."""
    wl = kvp_inputs.workload(1)
    li = kvp_inputs.make_layer(wl)
    q, kk = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, kk).cpu().numpy()
    exact = oracle.future_mass(li.q, li.k, wl.window, f32_exact=True)["lse"]
    rounded = oracle.future_mass(li.q, li.k, wl.window)["lse"]
    assert np.abs(lse - exact).max() < 1e-5 < np.abs(lse - rounded).max()


def test_f32_lse_with_one_dominant_key():
    """A row whose sink key dominates (a logit about 13 above the rest) over
    thousands of keys: each other term is below half an fp32 ulp of the
    running sum, so the sum is kept in fp64.  An fp32 sum loses those terms:
    2.8e-5 on this input (emulated on the CPU), 1e-4 on a 7.5K-key row of a
    64-head layer; the fp64 sum stays below 1e-6."""
    wl = kvp_inputs.workload(2).with_(B=1, Hq=2, Hkv=1, S=7886, D=128, window=100, n_sink=6,
                                      top_k=3660, dtype="f32", seed=4343)
    li = kvp_inputs.make_layer(wl)
    say("[f32] one dominant key: B=1 Hq=2 Hkv=1 S=7886 D=128")
    q, kk = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, kk)
    mass = kvp.future_mass(q, kk, lse, wl.window)
    torch.cuda.synchronize()
    ref = oracle.future_mass(li.q, li.k, wl.window, f32_exact=True)
    assert np.abs(lse.cpu().numpy() - ref["lse"]).max() <= 1e-5
    assert_mass(mass.cpu().numpy(), ref["mass"], "f32 mass, one dominant key")
