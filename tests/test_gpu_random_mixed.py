"""GPU parity on seeded random shapes that mix what the fixed cases keep
apart: fp32 or bf16 inputs (fp32 rounded to bf16 on load), d = 64 or 128,
batch sizes above one, GQA groups from 1 to 8, random window, sinks and
budget, query blocks of the Golden-Eviction scores per KV head or per query
head, and the sparse LSE over a running top-k pattern.  Every output is
compared in full with the oracle: LSE, group and per-head masses, block and
future scores, the static ranks and cutoffs (bit-exact) and the sparse LSE
(same pattern of empty rows, then within the LSE tolerance)."""
import numpy as np
import pytest
import torch

import future_attention_scoring_kvp_amd as kvp
import kvp_inputs
import oracle
from parity import LSE_ATOL, assert_lse, assert_mass, say, to_dev

pytestmark = pytest.mark.gpu

# (B, Hkv, G, S range): one query head; small ragged groups; a 4-wave grid;
# one-workgroup-per-CU grids with paired tiles (the next three); short grids
# of one 32-row block per wave with paired tiles in both passes (the last)
FAMILIES = [(1, 1, 1, 1, 700), (2, 2, 3, 33, 1500), (1, 8, 4, 1000, 3000), (3, 8, 1, 1, 600),
            (2, 32, 2, 3585, 4096), (1, 64, 1, 3585, 4096), (1, 16, 8, 1537, 2048),
            (2, 4, 4, 3841, 4096)]


@pytest.mark.parametrize("family", range(len(FAMILIES)))
def test_random_mixed_shapes(family):
    B, Hkv, G, lo, hi = FAMILIES[family]
    rng = np.random.default_rng(3100 + family)
    D = int(rng.choice([64, 128]))
    dtype = "f32" if family % 2 == 0 else "bf16"
    S = int(rng.integers(lo, hi + 1))
    Hq = Hkv * G
    w = int(rng.integers(0, max(2, S // 3)))
    s = int(rng.integers(0, 8))
    k = int(rng.integers(0, S + 5))
    L = int(rng.choice([32, 64, 128, 256]))
    start = int(rng.integers(0, S // 32 + 1)) * 32
    per_head = family % 3 == 1
    say(f"[random mixed] family {family}: B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} {dtype} w={w} "
        f"s={s} k={k} blocks {start}+{L} per_head={per_head}")
    wl = kvp_inputs.workload(2).with_(B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, window=w, n_sink=s,
                                      top_k=k, dtype=dtype, seed=31000 + family)
    li = kvp_inputs.make_layer(wl)
    pri = (np.round(rng.standard_normal((B, Hkv, S)) * 2) / 4).astype(np.float32)

    q, kk = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, kk)
    mass = kvp.future_mass(q, kk, lse, w)
    ph = kvp.future_mass_per_head(q, kk, lse, w)
    blk, fut = kvp.block_future_scores(q, kk, lse, start, L, window=w, per_head=per_head)
    rank, cut = kvp.running_cutoff(to_dev(pri), w, s, k)
    lsp = kvp.lse_sparse(q, kk, rank, cut, w)
    torch.cuda.synchronize()

    what = f"family {family}"
    exact = dtype == "f32"   # fp32 inputs are used as given (no bf16 rounding)
    ref = oracle.future_mass(li.q, li.k, w, want_per_head=True, f32_exact=exact)
    assert_lse(lse.cpu().numpy(), ref["lse"], what)
    assert_mass(mass.cpu().numpy(), ref["mass"], what)
    assert_mass(ph.cpu().numpy(), ref["mass_heads"], what + " per head")
    if blk.shape[2] > 0:
        rb = oracle.block_scores(li.q, li.k, w, start, L, per_head=per_head, f32_exact=exact)
        assert_mass(blk.cpu().numpy(), rb["block"], what + " block")
        assert_mass(fut.cpu().numpy(), rb["future"], what + " future")

    r_rank, r_cut = oracle.running_cutoff(pri.astype(np.float64), w, s, k)
    assert np.array_equal(rank.cpu().numpy(), r_rank), what + " rank"
    assert np.array_equal(cut.cpu().numpy(), r_cut), what + " cutoff"
    r_sp = oracle.sparse_lse(li.q, li.k, w, r_rank, r_cut, f32_exact=exact)
    got = lsp.cpu().numpy().astype(np.float64)
    finite = np.isfinite(r_sp)
    assert np.array_equal(finite, np.isfinite(got)), what + " sparse LSE: empty rows differ"
    if finite.any():
        err = np.abs(got[finite] - r_sp[finite]).max()
        assert err <= LSE_ATOL, f"{what} sparse LSE: max |d| {err:.3g}"
