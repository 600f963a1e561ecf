"""GPU parity of the running top-k sparse log-normaliser (KVpop §3.2: the
student's sparse attention keeps the sinks, the protected window and the
top-k eligible tokens; its per-query LSE replaces the dense one in the
target) against the CPU oracle."""
import math

import numpy as np
import pytest
import torch

import future_attention_scoring_kvp_amd as kvp
import kvp_inputs
import oracle
from parity import LSE_ATOL, say, to_dev

pytestmark = pytest.mark.gpu


def priorities(rng, B, Hkv, S):
    return (np.round(rng.standard_normal((B, Hkv, S)) * 2) / 4).astype(np.float32)


@pytest.mark.parametrize("B,Hq,Hkv,S,D,w,s,k,dtype", [
    (1, 4, 1, 300, 128, 20, 4, 32, "bf16"),
    (2, 8, 2, 1000, 128, 64, 4, 100, "bf16"),
    (1, 4, 4, 257, 64, 0, 3, 40, "bf16"),          # no window
    (1, 8, 1, 2100, 128, 512, 4, 1024, "bf16"),    # many blocks outside every window
    (1, 1, 1, 256, 64, 16, 4, 32, "f32"),          # fp32 inputs, exact fp32 path
    (2, 8, 2, 1000, 128, 40, 4, 100, "f32"),
    (1, 4, 2, 200, 128, 8, 2, 10_000, "bf16"),     # full budget: the dense LSE
    (1, 32, 8, 8100, 128, 512, 4, 2000, "bf16"),   # one-per-CU grid with paired tiles
])
def test_sparse_lse_matches_oracle(B, Hq, Hkv, S, D, w, s, k, dtype):
    wl = kvp_inputs.workload(2).with_(B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype=dtype, seed=900 + S)
    li = kvp_inputs.make_layer(wl)
    rng = np.random.default_rng(S + k)
    say(f"[sparse lse] B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} w={w} s={s} k={k} {dtype}")
    q, kt = to_dev(li.q), to_dev(li.k)
    rank, cut = kvp.running_cutoff(to_dev(priorities(rng, B, Hkv, S)), w, s, k)
    lse = kvp.lse_sparse(q, kt, rank, cut, w)
    torch.cuda.synchronize()
    ref = oracle.sparse_lse(li.q, li.k, w, rank.cpu().numpy(), cut.cpu().numpy(),
                            f32_exact=dtype == "f32")
    got = lse.cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    assert err.max() <= LSE_ATOL, f"max |d| {err.max():.3g} at {np.unravel_index(err.argmax(), err.shape)}"
    if k >= S:
        dense = kvp.lse_fwd(q, kt)
        torch.cuda.synchronize()
        assert (lse - dense).abs().max().item() <= LSE_ATOL


def test_empty_pattern_is_minus_inf():
    wl = kvp_inputs.workload(2).with_(Hq=4, Hkv=1, S=128, D=128, seed=4)
    li = kvp_inputs.make_layer(wl)
    q, kt = to_dev(li.q), to_dev(li.k)
    rank, cut = kvp.running_cutoff(torch.zeros(1, 1, 128, device="cuda"), 0, 0, 0)
    lse = kvp.lse_sparse(q, kt, rank, cut, 0)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(lse))


def test_full_length_layer_sampled_rows_and_target():
    """Qwen3-4B-shaped layer (32/8 heads, S = 32768), priorities from the GPU's
    own KVpop target scores, window 512, 4 sinks, k = 16384: sampled rows
    against an fp64 recomputation from the definition; then the mass pass
    on the sparse LSE (the page's target), which bounds the dense mass from
    above since the sparse normaliser is smaller."""
    wl = kvp_inputs.workload(4).with_(layers=1)
    li = kvp_inputs.make_layer(wl)
    w, s, k, S, D, G = wl.window, wl.n_sink, wl.top_k, wl.S, wl.D, wl.G
    say(f"[sparse lse] full length S={S}")
    q, kt = to_dev(li.q), to_dev(li.k)
    lse_d = kvp.lse_fwd(q, kt)
    score = kvp.target_scores(kvp.future_mass_per_head(q, kt, lse_d, w), wl.Hkv, w)
    rank, cut = kvp.running_cutoff(score, w, s, k)
    lse_s = kvp.lse_sparse(q, kt, rank, cut, w)
    mass_s = kvp.future_mass(q, kt, lse_s, w)
    mass_d = kvp.future_mass(q, kt, lse_d, w)
    torch.cuda.synchronize()
    rk, ct = rank.cpu().numpy(), cut.cpu().numpy()
    got = lse_s.cpu().numpy()
    qf, kf = li.q_f32(), li.k_f32()
    rows = [0, 1, 5, 511, 512, 513, 600, 4096, 16383, 16384, 16900, 30000, 32767]
    for g in (0, 13):
        h = g // G
        for i in rows:
            j = np.arange(i + 1)
            keep = ((i - j) < w) | (rk[0, h, j] <= ct[0, h, i])
            logits = kf[0, h, j][keep].astype(np.float64) @ qf[0, g, i].astype(np.float64) / math.sqrt(D)
            m = logits.max()
            ref = m + math.log(np.exp(logits - m).sum())
            assert abs(got[0, g, i] - ref) <= LSE_ATOL, (g, i, got[0, g, i], ref)
    assert torch.all(lse_s <= lse_d + LSE_ATOL)
    assert torch.all(torch.isfinite(mass_s))
    assert torch.all(mass_s >= mass_d * (1 - 1e-4) - 1e-6)
