"""Rows whose shifted exponential sum leaves the fp32 range, on the bf16
matrix-core path.  The LSE kernels shift each row by the largest logit of its
first key block, so a later key whose logit exceeds that shift by more than
about 88 (natural units) flags the row, and the rows so flagged are recomputed
exactly by a max-then-sum pass.  Here one key has a huge logit for the query
heads whose queries are all positive, and ordinary ones for the others, so
flagged and unflagged rows sit side by side in every launch shape of the dense
LSE (4-wave, 8-wave paired one-block, two- and three-block grids) and of the
sparse LSE (the running top-k pattern of KVpop §3.2).  The LSE (LKV §3 Eq. 1,
the per-query log-normaliser reused by KVpop §3.2 Eq. 8) and the future mass
(KVpop §3.1 Eq. 2, un-normalised as in App. B.1) are compared element by
element with the oracle."""
import numpy as np
import pytest
import torch

import future_attention_scoring_kvp_amd as kvp
import kvp_inputs
import oracle
from parity import LSE_ATOL, assert_mass, say, to_dev

pytestmark = pytest.mark.gpu

BF16_BIG = {128: 0x41A0, 64: 0x41F0}   # 20.0 and 30.0 as bf16 bit patterns


def layer_with_huge_key(B, Hq, Hkv, S, D, j_big, seed):
    """A bf16 layer of N(0,1) inputs where K row j_big of every KV head is a
    large constant and the queries of the even query heads are made positive
    (sign bit cleared): their logits against that key exceed the first key
    block's by far more than the fp32 exponent range."""
    wl = kvp_inputs.workload(2).with_(B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, seed=seed)
    li = kvp_inputs.make_layer(wl)
    li.q[:, 0::2] &= np.uint16(0x7FFF)
    li.k[:, :, j_big, :] = np.uint16(BF16_BIG[D])
    return li


def check_flagged(ref_lse, h_heads, j_big):
    """The test's own construction: the rows at and after the huge key of the
    positive-query heads have an LSE above 130, while no first-block logit of
    these N(0,1) inputs comes near 40, so each such row leaves the range."""
    flagged = ref_lse[:, h_heads, j_big:]
    assert np.all(flagged > 130.0), "construction did not push the rows out of range"


@pytest.mark.parametrize("B,Hq,Hkv,S,D,j_big,launch", [
    (1, 4, 1, 300, 128, 200, "4-wave, two blocks"),
    (2, 4, 2, 333, 64, 40, "4-wave, two blocks, d = 64"),
    (1, 32, 8, 4096, 128, 1000, "8-wave paired, one block"),
    (1, 32, 8, 8192, 128, 5000, "8-wave, two blocks"),
    (1, 32, 8, 16384, 128, 16000, "8-wave, three blocks"),
])
def test_dense_lse_flagged_rows(B, Hq, Hkv, S, D, j_big, launch):
    li = layer_with_huge_key(B, Hq, Hkv, S, D, j_big, seed=4242 + S + D)
    w = 64
    say(f"[lse fallback] {launch}: B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} key {j_big}")
    q, k = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, k)
    mass = kvp.future_mass(q, k, lse, w)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(lse))
    G = Hq // Hkv
    got_lse, got_mass = lse.cpu().numpy(), mass.cpu().numpy()
    # small shapes in full; larger ones on the first and last KV head
    units = [(b, h) for b in range(B) for h in range(Hkv)] if S <= 1000 else \
        [(0, 0), (B - 1, Hkv - 1)]
    for b, h in units:
        ref = oracle.future_mass(li.q, li.k, w, b_only=b, h_only=h)
        heads = slice(h * G, (h + 1) * G)
        check_flagged(ref["lse"][b:b + 1, heads], slice(0, None, 2), j_big)
        err = np.abs(got_lse[b, heads] - ref["lse"][b, heads])
        assert err.max() <= LSE_ATOL, \
            f"b={b} h={h}: max |d| {err.max():.3g} at {np.unravel_index(err.argmax(), err.shape)}"
        assert_mass(got_mass[b, h], ref["mass"][b, h], f"{launch} b={b} h={h}")


@pytest.mark.parametrize("B,Hq,Hkv,S,D,j_big", [
    (1, 4, 1, 300, 128, 200),
    (1, 32, 8, 8192, 128, 3000),   # 8-wave grid
])
def test_sparse_lse_flagged_rows(B, Hq, Hkv, S, D, j_big):
    """The huge key is given the highest priority, so every row after it keeps
    it in its pattern and overflows."""
    li = layer_with_huge_key(B, Hq, Hkv, S, D, j_big, seed=5151 + S)
    w, s, top = 32, 4, max(8, S // 8)
    rng = np.random.default_rng(S)
    prio = (np.round(rng.standard_normal((B, Hkv, S)) * 2) / 4).astype(np.float32)
    prio[:, :, j_big] = 100.0
    say(f"[lse fallback] sparse B={B} Hq={Hq} Hkv={Hkv} S={S} key {j_big}")
    q, k = to_dev(li.q), to_dev(li.k)
    rank, cut = kvp.running_cutoff(to_dev(prio), w, s, top)
    lse = kvp.lse_sparse(q, k, rank, cut, w)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(lse))
    rk, ct = rank.cpu().numpy(), cut.cpu().numpy()
    G = Hq // Hkv
    if S <= 1000:
        ref = oracle.sparse_lse(li.q, li.k, w, rk, ct)
        check_flagged(ref, slice(0, None, 2), j_big)
        err = np.abs(lse.cpu().numpy() - ref)
        assert err.max() <= LSE_ATOL, f"max |d| {err.max():.3g}"
    else:
        # the first KV head's query heads: the oracle on that head's slice
        h = 0
        ref = oracle.sparse_lse(li.q[:, :G], li.k[:, :1], w, rk[:, :1], ct[:, :1])
        check_flagged(ref, slice(0, None, 2), j_big)
        err = np.abs(lse.cpu().numpy()[:, h * G:(h + 1) * G] - ref)
        assert err.max() <= LSE_ATOL, f"max |d| {err.max():.3g}"
