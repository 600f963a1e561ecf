"""GPU parity of the Golden-Eviction block and future scores (ForesightKV,
§3.2 "Golden Eviction"; the appendix's block surrogate) against the CPU
oracle, plus full-length checks on sampled keys and the identity with the
future mass."""
import math

import numpy as np
import pytest
import torch

import future_attention_scoring_kvp_amd as kvp
import kvp_inputs
import oracle
from parity import MASS_ATOL, MASS_RTOL, say, to_dev

pytestmark = pytest.mark.gpu


def block_tol(ref, counts, G):
    """The mass tolerance on the un-normalised block sums, carried to the
    means: |d| <= (1e-5 + 2e-3 |sum|) / (G |Q_t|)."""
    c = (counts * G)[None, None, :, None]
    return MASS_ATOL / c + MASS_RTOL * np.abs(ref)


def assert_blocks(got, ref, counts, G, what):
    got = got.astype(np.float64)
    bad = np.abs(got - ref) > block_tol(ref, counts, G)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance, first at "
                           f"{np.argwhere(bad)[0].tolist()}: {got[bad][:3]} vs {ref[bad][:3]}")


def counts_of(S, start, L):
    nb = kvp.block_count(S, start, L)
    return np.array([min(L, S - start - t * L) for t in range(nb)], dtype=np.float64)


@pytest.mark.parametrize("B,Hq,Hkv,S,D,w,start,L,per_head,dtype", [
    (1, 4, 1, 300, 128, 0, 32, 64, False, "bf16"),    # ragged last block
    (2, 8, 2, 1000, 128, 0, 64, 128, False, "bf16"),
    (2, 8, 2, 1000, 128, 0, 64, 128, True, "bf16"),   # per query head
    (1, 4, 4, 257, 64, 5, 0, 32, False, "bf16"),      # d = 64, window, blocks from row 0
    (1, 8, 1, 2100, 128, 0, 1024, 256, False, "bf16"),  # first block after 1024 rows
    (1, 2, 1, 200, 128, 0, 0, 512, False, "bf16"),    # one block longer than S
    (1, 1, 1, 256, 64, 0, 32, 32, False, "f32"),      # fp32 inputs, exact fp32 path
    (2, 8, 2, 700, 128, 40, 64, 96, True, "f32"),
])
def test_block_scores_match_oracle(B, Hq, Hkv, S, D, w, start, L, per_head, dtype):
    wl = kvp_inputs.workload(2).with_(B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, dtype=dtype, seed=500 + S)
    li = kvp_inputs.make_layer(wl)
    say(f"[block] B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} w={w} start={start} L={L} "
        f"per_head={per_head} {dtype}")
    q, k = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, k)
    blk, fut = kvp.block_future_scores(q, k, lse, start, L, w, per_head=per_head)
    _, fut_only = kvp.block_future_scores(q, k, lse, start, L, w, per_head=per_head,
                                          want_block=False)
    torch.cuda.synchronize()
    ref = oracle.block_scores(li.q, li.k, w, start, L, per_head=per_head,
                              f32_exact=dtype == "f32")
    counts = counts_of(S, start, L)
    G = 1 if per_head else Hq // Hkv
    assert_blocks(blk.cpu().numpy(), ref["block"], counts, G, "block scores")
    assert_blocks(fut.cpu().numpy(), ref["future"], counts, G, "future scores")
    # the future scores do not depend on whether the block scores are written
    assert torch.equal(fut, fut_only)
    # on the GPU's own block scores the future score is exactly their suffix max
    own = torch.flip(torch.cummax(torch.flip(blk, [2]), 2).values, [2])
    assert torch.equal(fut, own)


def test_no_block_and_deterministic():
    wl = kvp_inputs.workload(2).with_(Hq=8, Hkv=2, S=512, seed=77)
    li = kvp_inputs.make_layer(wl)
    q, k = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, k)
    blk, fut = kvp.block_future_scores(q, k, lse, 512, 64)
    assert blk.shape == (1, 2, 0, 512) and fut.shape == (1, 2, 0, 512)
    a = kvp.block_future_scores(q, k, lse, 96, 64)
    b = kvp.block_future_scores(q, k, lse, 96, 64)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_full_length_layer_sampled_keys():
    """Qwen3-4B-shaped layer (32/8 heads, S = 32768), blocks of 256 rows after
    1024 (the budget and eviction length ForesightKV trains with): sampled
    keys against an fp64 recomputation p = exp(scale <q_i, k_j> - LSE_i)
    from the GPU's LSE (itself checked against the oracle elsewhere), and
    every key from the first block start on against the GPU's future mass
    (which then counts exactly the rows of the blocks)."""
    wl = kvp_inputs.workload(4).with_(layers=1)
    li = kvp_inputs.make_layer(wl)
    start, L, S, D, G = 1024, 256, wl.S, wl.D, wl.G
    say(f"[block] full length S={S} start={start} L={L}")
    q, k = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, k)
    blk, fut = kvp.block_future_scores(q, k, lse, start, L)
    mass = kvp.future_mass(q, k, lse, 0)
    torch.cuda.synchronize()
    counts = counts_of(S, start, L)
    nb = len(counts)
    blk_np, fut_np = blk.cpu().numpy(), fut.cpu().numpy()
    lse_np = lse.cpu().numpy().astype(np.float64)
    qf, kf = li.q_f32(), li.k_f32()
    rng = np.random.default_rng(5)
    keys = sorted({0, 1, 511, 512, 1023, 1024, 1279, 1280, 16383, 16384, 32511, 32512, 32767,
                   *rng.integers(0, S, 8).tolist()})
    scale = 1.0 / math.sqrt(D)
    for h in (0, 5):
        ref_blk = np.zeros((nb, len(keys)))
        for gg in range(G):
            g = h * G + gg
            qg = qf[0, g, start:].astype(np.float64)
            logits = qg @ kf[0, h, keys].astype(np.float64).T * scale     # [S - start, n_keys]
            rows = np.arange(start, S)[:, None]
            p = np.where(rows >= np.array(keys)[None, :], np.exp(logits - lse_np[0, g, start:, None]), 0.0)
            pad = nb * L - p.shape[0]
            p = np.concatenate([p, np.zeros((pad, len(keys)))], 0)
            ref_blk += p.reshape(nb, L, len(keys)).sum(1)
        ref_blk /= counts[:, None] * G
        ref_fut = np.flip(np.maximum.accumulate(np.flip(ref_blk, 0), axis=0), 0)
        got_b = blk_np[0, h][:, keys].astype(np.float64)
        got_f = fut_np[0, h][:, keys].astype(np.float64)
        tol = MASS_ATOL / (counts[:, None] * G) + MASS_RTOL * np.abs(ref_blk)
        assert np.all(np.abs(got_b - ref_blk) <= tol), f"head {h}: block scores off"
        tolf = MASS_ATOL / (counts[:, None] * G) + MASS_RTOL * np.abs(ref_fut)
        assert np.all(np.abs(got_f - ref_fut) <= tolf), f"head {h}: future scores off"
    # summed over the blocks, keys j >= start see exactly the rows of the mass
    total = (blk.double() * torch.from_numpy(counts).cuda()[None, None, :, None]).sum(2) * G
    m = mass.double()
    rel = ((total[..., start:] - m[..., start:]).abs() / (m[..., start:].abs() + 1e-6)).max().item()
    assert rel < 1e-4, rel
