"""GPU parity of the chunked future-mass pass (kvp_future_mass_chunked): short
sequences whose 512-key tiles have their query sweeps cut into chunks, one
workgroup each, the partial masses added per key in chunk order through the
caller's workspace.  The masses are KVpop §3.1 Eq. 2 (un-normalised, App.
B.1), recovered from the LSE as in §3.2 Eq. 8, summed over the group or per
query head; they are compared element by element with the oracle, on the
4K-token GQA layer in full and on ragged shapes (odd group, d = 64, batches,
one and several rounds of chunks), and the chunked results are checked to be
bitwise reproducible, independent of the workspace's previous contents, and
within the tolerance of the unchunked pass.  Per-head masses are not chunked
(the call runs the per-head launch); they are checked here too."""
import numpy as np
import pytest
import torch

import future_attention_scoring_kvp_amd as kvp
import kvp_inputs
import oracle
from parity import assert_mass, say, to_dev

pytestmark = pytest.mark.gpu


def run(li, w, per_head, ws=None):
    q, k = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, k)
    need = kvp.future_mass_workspace_bytes(q, k, w, per_head)
    assert need > 0, "the shape must take the chunked launch"
    m = kvp.future_mass_chunked(q, k, lse, w, per_head=per_head, workspace=ws)
    torch.cuda.synchronize()
    return q, k, lse, m


def test_gqa4k_layer_whole():
    """The 4K-token GQA layer (32/8 heads, w = 128): every key of every head,
    group sums and per-head masses."""
    wl = kvp_inputs.workload(2)
    li = kvp_inputs.make_layer(wl)
    say("[chunked] 4K layer: GPU path")
    q, k, lse, m = run(li, wl.window, False)
    mh = kvp.future_mass_chunked(q, k, lse, wl.window, per_head=True)
    torch.cuda.synchronize()
    say("[chunked] 4K layer: oracle")
    ref = oracle.future_mass(li.q, li.k, wl.window, want_per_head=True)
    assert_mass(m.cpu().numpy(), ref["mass"], "4K chunked group")
    assert_mass(mh.cpu().numpy(), ref["mass_heads"], "4K chunked per head")
    assert np.all(m.cpu().numpy()[:, :, wl.S - wl.window:] == 0)


@pytest.mark.parametrize("B,Hq,Hkv,S,w,D", [
    (2, 16, 4, 3990, 100, 128),   # S % 32 = 22: a partial last query block
    (2, 16, 4, 3990, 100, 64),
    (1, 24, 8, 8100, 257, 128),   # odd group; several rounds of chunks
    (1, 4, 1, 1000, 10, 128),     # one-block chunks
    (3, 6, 3, 2049, 0, 64),       # H2O (w = 0), S = 4 tiles + 1 key
])
def test_ragged_shapes(B, Hq, Hkv, S, w, D):
    wl = kvp_inputs.workload(2).with_(B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, window=w,
                                      seed=6161 + S + D + Hq)
    li = kvp_inputs.make_layer(wl)
    say(f"[chunked] B={B} Hq={Hq} Hkv={Hkv} S={S} w={w} D={D}")
    q, k, lse, m = run(li, w, False)
    mh = kvp.future_mass_chunked(q, k, lse, w, per_head=True)
    torch.cuda.synchronize()
    G = Hq // Hkv
    for b, h in ((0, 0), (B - 1, Hkv - 1)):
        ref = oracle.future_mass(li.q, li.k, w, b_only=b, h_only=h, want_per_head=True)
        assert_mass(m.cpu().numpy()[b, h], ref["mass"][b, h], f"S={S} group b={b} h={h}")
        assert_mass(mh.cpu().numpy()[b, h * G:(h + 1) * G], ref["mass_heads"][b, h * G:(h + 1) * G],
                    f"S={S} per head b={b} h={h}")
    # every unit: the w = 0 row sums, and the group sum of the per-head masses
    m0 = kvp.future_mass_chunked(q, k, lse, 0).double().sum(dim=2).cpu().numpy()
    np.testing.assert_allclose(m0, G * S, rtol=1e-4)
    np.testing.assert_allclose(mh.cpu().numpy().reshape(B, Hkv, G, S).astype(np.float64).sum(2),
                               m.cpu().numpy(), rtol=1e-5, atol=1e-6)


def test_reproducible_and_workspace_independent():
    """Two calls give the same bits; a workspace filled with garbage, reused by
    a call with other chunks, changes nothing; the unchunked pass agrees within
    the tolerance."""
    wl = kvp_inputs.workload(2)
    li = kvp_inputs.make_layer(wl)
    q, k = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, k)
    need = kvp.future_mass_workspace_bytes(q, k, wl.window)
    ws = torch.full((need + 4096,), 0x7F, dtype=torch.uint8, device="cuda")   # NaN patterns
    a = kvp.future_mass_chunked(q, k, lse, wl.window, workspace=ws)
    b = kvp.future_mass_chunked(q, k, lse, wl.window, workspace=ws)
    # a shorter window: other chunks over the same, now dirty, workspace
    w2 = wl.window // 2
    assert kvp.future_mass_workspace_bytes(q, k, w2) <= ws.numel()
    c1 = kvp.future_mass_chunked(q, k, lse, w2, workspace=ws)
    c2 = kvp.future_mass_chunked(q, k, lse, w2)
    plain = kvp.future_mass(q, k, lse, wl.window)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(c1, c2)
    assert torch.isfinite(a).all() and torch.isfinite(c1).all()
    assert_mass(a.cpu().numpy(), plain.cpu().numpy().astype(np.float64), "chunked vs unchunked")


def test_long_sequences_per_head_and_fp32_take_the_plain_launch():
    """Where the grid is already full, for per-head masses and for fp32 input
    the size is 0 and the call (with no workspace) gives the unchunked pass's
    bits."""
    wl = kvp_inputs.workload(4).with_(B=2, S=16384, window=256, seed=77)   # 2 x 8 x 32 tiles
    li = kvp_inputs.make_layer(wl)
    q, k = to_dev(li.q), to_dev(li.k)
    assert kvp.future_mass_workspace_bytes(q, k, wl.window) == 0
    lse = kvp.lse_fwd(q, k)
    a = kvp.future_mass_chunked(q, k, lse, wl.window)
    b = kvp.future_mass(q, k, lse, wl.window)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    wl2 = kvp_inputs.workload(2)
    li2 = kvp_inputs.make_layer(wl2)
    q2, k2 = to_dev(li2.q), to_dev(li2.k)
    assert kvp.future_mass_workspace_bytes(q2, k2, wl2.window, True) == 0
    lse2 = kvp.lse_fwd(q2, k2)
    c = kvp.future_mass_chunked(q2, k2, lse2, wl2.window, per_head=True)
    d = kvp.future_mass_per_head(q2, k2, lse2, wl2.window)
    torch.cuda.synchronize()
    assert torch.equal(c, d)
    # fp32 input (the tiny workload) keeps its exact fp32 launch
    wl1 = kvp_inputs.workload(1)
    li1 = kvp_inputs.make_layer(wl1)
    q1, k1 = to_dev(li1.q), to_dev(li1.k)
    assert kvp.future_mass_workspace_bytes(q1, k1, wl1.window) == 0
    lse1 = kvp.lse_fwd(q1, k1)
    e = kvp.future_mass_chunked(q1, k1, lse1, wl1.window)
    f = kvp.future_mass(q1, k1, lse1, wl1.window)
    torch.cuda.synchronize()
    assert torch.equal(e, f)


@pytest.mark.parametrize("seed", range(6))
def test_random_short_shapes(seed):
    """Seeded random short shapes (any grid the chunk plan makes: one to four
    rounds, tiles with no future query, ragged S and windows), one unit
    against the oracle and every unit through the w = 0 identity."""
    rng = np.random.default_rng(9900 + seed)
    B = int(rng.integers(1, 4))
    Hkv = int(rng.integers(1, 9))
    G = int(rng.integers(1, 5))
    S = int(rng.integers(33, 9001))
    D = int(rng.choice([64, 128]))
    w = int(rng.integers(0, S // 2 + 1))
    wl = kvp_inputs.workload(2).with_(B=B, Hq=Hkv * G, Hkv=Hkv, S=S, D=D, window=w,
                                      seed=9900 + seed)
    li = kvp_inputs.make_layer(wl)
    q, k = to_dev(li.q), to_dev(li.k)
    need = kvp.future_mass_workspace_bytes(q, k, w)
    say(f"[chunked] random {seed}: B={B} Hkv={Hkv} G={G} S={S} D={D} w={w} workspace={need}")
    lse = kvp.lse_fwd(q, k)
    m = kvp.future_mass_chunked(q, k, lse, w)
    m0 = kvp.future_mass_chunked(q, k, lse, 0).double().sum(dim=2).cpu().numpy()
    torch.cuda.synchronize()
    b, h = B - 1, int(rng.integers(0, Hkv))
    ref = oracle.future_mass(li.q, li.k, w, b_only=b, h_only=h)
    assert_mass(m.cpu().numpy()[b, h], ref["mass"][b, h], f"random {seed} b={b} h={h}")
    assert np.all(m.cpu().numpy()[:, :, S - w:] == 0)
    np.testing.assert_allclose(m0, G * S, rtol=1e-4)


@pytest.mark.parametrize("S,w", [(1, 0), (2, 1), (31, 0), (32, 5), (33, 0), (257, 16), (600, 599)])
def test_tiny_and_degenerate(S, w):
    """Sequences of one to a few hundred tokens, windows up to S - 1: the whole
    output against the oracle."""
    wl = kvp_inputs.workload(2).with_(B=2, Hq=4, Hkv=2, S=S, D=64, window=w, seed=77 + S + w)
    li = kvp_inputs.make_layer(wl)
    q, k = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, k)
    m = kvp.future_mass_chunked(q, k, lse, w)
    torch.cuda.synchronize()
    ref = oracle.future_mass(li.q, li.k, w)
    assert_mass(m.cpu().numpy(), ref["mass"], f"S={S} w={w}")
