"""GPU parity for the grids that give each workgroup two tiles: in the mass
pass a workgroup sweeps key tile m with the query blocks descending and then
key tile T-1-m with them ascending; in the LSE pass it takes the tile of the
longest rows and then the tile of the shortest.  These grids are chosen for
one-workgroup-per-CU launches, so the shapes are Qwen3-4B-sized (32 query /
8 KV heads, d = 128, S near 32K): an odd number of key tiles (the middle tile
has no partner), and a sequence that is not a multiple of 32 (a partial last
query block, masked in both sweep directions).  Two whole units per shape are
compared with the oracle, for the group sums and the per-head masses; every
unit is checked through the w = 0 row-sum identity.  The query-block mode
(Golden-Eviction scores) is checked on the same shapes, group and per head,
against the oracle-checked masses: with blocks from row 0 the block means
times their row and head counts add up to the mass, and the future score is
the running maximum of the block scores from the end (exact); the attribution
to blocks is checked against the oracle's mass from the last blocks' rows."""
import numpy as np
import pytest
import torch

import future_attention_scoring_kvp_amd as kvp
import kvp_inputs
import oracle
from parity import assert_keep, assert_lse, assert_mass, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("S,w,D", [
    (32000, 77, 128),    # 63 key tiles of 512: tile 31 sweeps alone; S % 512 = 256
    (32749, 300, 128),   # 64 key tiles, the last one partial; S % 32 = 13
    (32749, 300, 64),    # the same at d = 64 (four 16-wide slices per operand)
])
def test_paired_tiles(S, w, D):
    wl = kvp_inputs.workload(4).with_(S=S, D=D, window=w, seed=4242 + S + D)
    say(f"[paired] S={S} w={w} D={D}: generating inputs")
    li = kvp_inputs.make_layer(wl)
    q, k = to_dev(li.q), to_dev(li.k)
    say(f"[paired] S={S} w={w}: GPU path")
    lse = kvp.lse_fwd(q, k)
    mass = kvp.future_mass(q, k, lse, w)
    per_head = kvp.future_mass_per_head(q, k, lse, w)
    total0 = kvp.future_mass(q, k, lse, 0).double().sum(dim=2)
    torch.cuda.synchronize()
    lse_h, mass_h, ph_h = lse.cpu().numpy(), mass.cpu().numpy(), per_head.cpu().numpy()
    G = wl.G
    assert np.all(mass_h[:, :, S - w:] == 0)
    # w = 0: every softmax row sums to one, so each KV head's total is G * S
    np.testing.assert_allclose(total0.cpu().numpy(), G * S, rtol=1e-4)
    # the group sum is the sum of its heads' masses
    np.testing.assert_allclose(ph_h.reshape(1, wl.Hkv, G, S).astype(np.float64).sum(axis=2),
                               mass_h, rtol=1e-5, atol=1e-6)
    check_blocks(q, k, lse, S, w, G, mass_h, ph_h, li)
    for h in (0, wl.Hkv - 1):
        say(f"[paired] S={S} w={w}: oracle unit h={h}")
        ref = oracle.future_mass(li.q, li.k, w, b_only=0, h_only=h, want_per_head=True)
        g0 = h * G
        assert_lse(lse_h[0, g0:g0 + G], ref["lse"][0, g0:g0 + G], f"paired S={S} lse h={h}")
        assert_mass(mass_h[0, h], ref["mass"][0, h], f"paired S={S} mass h={h}")
        assert_mass(ph_h[0, g0:g0 + G], ref["mass_heads"][0, g0:g0 + G],
                    f"paired S={S} per-head h={h}")


def check_blocks(q, k, lse, S, w, G, mass_h, ph_h, li):
    wl_kv = li.wl.Hkv
    L = 1024                      # blocks [0, 1024), ..., the last one partial
    n = kvp.block_count(S, 0, L)
    rows = np.array([min(S, (t + 1) * L) - t * L for t in range(n)], np.float64)
    for per_head, ref, heads in ((False, mass_h, G), (True, ph_h, 1)):
        say(f"[paired] S={S} w={w}: block scores per_head={per_head}")
        blk, fut = kvp.block_future_scores(q, k, lse, 0, L, window=w, per_head=per_head)
        torch.cuda.synchronize()
        blk, fut = blk.cpu().numpy(), fut.cpu().numpy()
        assert blk.shape[2] == n
        total = (blk.astype(np.float64) * (rows * heads)[None, None, :, None]).sum(axis=2)
        np.testing.assert_allclose(total, ref, rtol=2e-5, atol=1e-6)
        suffix = np.maximum.accumulate(blk[:, :, ::-1], axis=2)[:, :, ::-1]
        assert np.array_equal(fut, suffix), f"future scores S={S} per_head={per_head}"
        # attribution to blocks: the block sums from block t on are the mass
        # from rows >= t L only, which the oracle computes with row_lo
        h = wl_kv - 1
        for t in (n - 2, n - 1):
            say(f"[paired] S={S} w={w}: oracle rows >= {t * L}, unit h={h}, per_head={per_head}")
            ref_t = oracle.future_mass(li.q, li.k, w, b_only=0, h_only=h, row_lo=t * L,
                                       want_per_head=per_head)
            tail = (blk[0, :, t:].astype(np.float64) * (rows[t:] * heads)[None, :, None]).sum(axis=1)
            if per_head:
                assert_mass(tail[h * G:(h + 1) * G], ref_t["mass_heads"][0, h * G:(h + 1) * G],
                            f"block sums from {t} per head")
            else:
                assert_mass(tail[h], ref_t["mass"][0, h], f"block sums from {t}")


def test_paired_units_not_a_multiple_of_8():
    """12 KV heads: the paired grids (mass: 12 units x 64 pairs, three full
    rounds; LSE: 12 x 256 pairs) fall back to unit-major order over the whole
    grid instead of per XCD.  The oracle computes the tail rows of one unit
    (exact masses for the keys they cover) and sampled LSE rows of every head;
    every unit is checked through the w = 0 row-sum identity."""
    S, w = 65536, 256
    wl = kvp_inputs.workload(4).with_(Hq=48, Hkv=12, S=S, window=w, seed=1212)
    say(f"[paired] 48/12 heads S={S}: generating inputs")
    li = kvp_inputs.make_layer(wl)
    q, k = to_dev(li.q), to_dev(li.k)
    say(f"[paired] 48/12 heads S={S}: GPU path")
    lse = kvp.lse_fwd(q, k)
    mass = kvp.future_mass(q, k, lse, w)
    total0 = kvp.future_mass(q, k, lse, 0).double().sum(dim=2)
    torch.cuda.synchronize()
    np.testing.assert_allclose(total0.cpu().numpy(), wl.G * S, rtol=1e-4)
    lse_h, mass_h = lse.cpu().numpy(), mass.cpu().numpy()
    rng = np.random.default_rng(5)
    rows = np.stack([np.zeros(64, np.int64), rng.integers(0, wl.Hq, 64), rng.integers(0, S, 64)], 1)
    rows[:4, 2] = S - 1 - np.arange(4)
    say(f"[paired] 48/12 heads S={S}: oracle LSE rows")
    ref_rows = oracle.lse_rows(li.q, li.k, rows)
    assert np.abs(lse_h[0, rows[:, 1], rows[:, 2]] - ref_rows).max() <= 1e-4
    h, row_lo = 11, S - 1024
    say(f"[paired] 48/12 heads S={S}: oracle tail rows >= {row_lo} of h={h}")
    ref = oracle.future_mass(li.q, li.k, w, b_only=0, h_only=h, row_lo=row_lo)
    g0 = h * wl.G
    assert_lse(lse_h[0, g0:g0 + wl.G, row_lo:], ref["lse"][0, g0:g0 + wl.G, row_lo:], "48/12 tail")
    assert_mass(mass_h[0, h, row_lo - w:], ref["mass"][0, h, row_lo - w:], "48/12 tail")


@pytest.mark.parametrize("family", range(6))
def test_paired_random_shapes(family):
    """One seeded case per family of shapes whose one-tile 8-wave grids reach
    512 blocks with tile pairs filling whole rounds (the paired paths), with
    random window, sinks, budget, head dimension and query blocks; everything
    against the oracle in full: LSE, group and per-head masses, keep-sets,
    block and future scores."""
    B, Hkv, G, lo, hi = [(2, 64, 1, 1537, 2048), (1, 64, 1, 3585, 4096), (2, 32, 2, 3585, 4096),
                         (1, 32, 2, 7681, 8192), (4, 32, 1, 1537, 2048),
                         (1, 16, 8, 1537, 2048)][family]
    rng = np.random.default_rng(900 + family)
    D = int(rng.choice([64, 128]))
    S = int(rng.integers(lo, hi + 1))
    w = int(rng.integers(0, S // 3))
    s = int(rng.integers(0, 8))
    k = int(rng.integers(0, S + 5))
    L = int(rng.choice([32, 64, 128, 256]))
    start = int(rng.integers(0, S // 32)) * 32
    wl = kvp_inputs.workload(2).with_(B=B, Hq=Hkv * G, Hkv=Hkv, S=S, D=D, window=w, n_sink=s,
                                      top_k=k, seed=20000 + family)
    say(f"[paired] random family {family}: B={B} Hq={Hkv * G} Hkv={Hkv} S={S} D={D} w={w} "
        f"s={s} k={k} blocks {start}+{L}")
    li = kvp_inputs.make_layer(wl)
    q, kk = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, kk)
    mass = kvp.future_mass(q, kk, lse, w)
    ph = kvp.future_mass_per_head(q, kk, lse, w)
    keep = kvp.select_topk(mass, w, s, k)
    blk, fut = kvp.block_future_scores(q, kk, lse, start, L, window=w)
    torch.cuda.synchronize()
    ref = oracle.future_mass(li.q, li.k, w, want_per_head=True)
    what = f"random family {family}"
    assert_lse(lse.cpu().numpy(), ref["lse"], what)
    assert_mass(mass.cpu().numpy(), ref["mass"], what)
    assert_mass(ph.cpu().numpy(), ref["mass_heads"], what + " per head")
    assert_keep(keep.cpu().numpy(), ref["mass"], w, s, k, oracle.select(ref["mass"], w, s, k),
                what)
    rb = oracle.block_scores(li.q, li.k, w, start, L)
    assert_mass(blk.cpu().numpy(), rb["block"], what + " block")
    assert_mass(fut.cpu().numpy(), rb["future"], what + " future")


@pytest.mark.parametrize("B,Hq,Hkv,S,w,D", [
    # LSE: 63 tiles of 8 x 32 query rows per unit (the middle one alone);
    # mass: the group heads split in halves, 32 key tiles of 128; S % 32 = 22
    (2, 16, 4, 3990, 100, 128),
    (2, 16, 4, 3990, 100, 64),
    # odd tile counts: 31 key tiles of 128 (tile 15 alone), 61 LSE tiles
    (2, 16, 4, 3900, 64, 128),
    # odd group (no head split), 64 key tiles of 128 per KV head
    (1, 24, 8, 8100, 257, 128),
])
def test_one_block_per_wave_grids(B, Hq, Hkv, S, w, D):
    """Short sequences whose grids give every wave one 32-row block and every
    workgroup a long and a short tile (LSE: 8 waves of 32 query rows; mass: 4
    waves of 32 keys).  Two units against the oracle, every unit through the
    w = 0 row-sum identity and the per-head sums."""
    wl = kvp_inputs.workload(2).with_(B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, window=w,
                                      seed=5151 + S + D + Hq)
    say(f"[one block per wave] B={B} Hq={Hq} Hkv={Hkv} S={S} w={w} D={D}")
    li = kvp_inputs.make_layer(wl)
    q, k = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, k)
    mass = kvp.future_mass(q, k, lse, w)
    per_head = kvp.future_mass_per_head(q, k, lse, w)
    total0 = kvp.future_mass(q, k, lse, 0).double().sum(dim=2)
    torch.cuda.synchronize()
    lse_h, mass_h, ph_h = lse.cpu().numpy(), mass.cpu().numpy(), per_head.cpu().numpy()
    G = Hq // Hkv
    assert np.all(mass_h[:, :, S - w:] == 0)
    np.testing.assert_allclose(total0.cpu().numpy(), G * S, rtol=1e-4)
    np.testing.assert_allclose(ph_h.reshape(B, Hkv, G, S).astype(np.float64).sum(axis=2),
                               mass_h, rtol=1e-5, atol=1e-6)
    for b, h in ((0, 0), (B - 1, Hkv - 1)):
        say(f"[one block per wave] S={S} D={D}: oracle unit b={b} h={h}")
        ref = oracle.future_mass(li.q, li.k, w, b_only=b, h_only=h, want_per_head=True)
        g0 = h * G
        assert_lse(lse_h[b, g0:g0 + G], ref["lse"][b, g0:g0 + G], f"S={S} lse b={b} h={h}")
        assert_mass(mass_h[b, h], ref["mass"][b, h], f"S={S} mass b={b} h={h}")
        assert_mass(ph_h[b, g0:g0 + G], ref["mass_heads"][b, g0:g0 + G],
                    f"S={S} per-head b={b} h={h}")
