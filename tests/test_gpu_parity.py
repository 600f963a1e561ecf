"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Every test prints its case before touching the GPU."""
import numpy as np
import pytest
import torch

import future_attention_scoring_kvp_amd as kvp
import kvp_inputs
import oracle
from parity import (assert_keep, assert_lse, assert_mass, say, to_dev, MASS_ATOL, MASS_RTOL,
                    LSE_ATOL)

pytestmark = pytest.mark.gpu


def run_gpu(li, w, s, k, scale=0.0):
    q, kk = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, kk, scale=scale)
    mass = kvp.future_mass(q, kk, lse, w, scale=scale)
    keep = kvp.select_topk(mass, w, s, k)
    torch.cuda.synchronize()
    return lse.cpu().numpy(), mass.cpu().numpy(), keep.cpu().numpy()


def full_check(li, w, s, k, what, scale=0.0):
    say(f"[parity] {what}: B={li.wl.B} Hq={li.wl.Hq} Hkv={li.wl.Hkv} S={li.wl.S} D={li.wl.D} "
        f"{li.wl.dtype} w={w} s={s} k={k}")
    lse, mass, keep = run_gpu(li, w, s, k, scale)
    ref = oracle.future_mass(li.q, li.k, w, scale=scale, f32_exact=li.wl.dtype == "f32")
    assert_lse(lse, ref["lse"], what)
    assert_mass(mass, ref["mass"], what)
    exact = oracle.select(ref["mass"], w, s, k)
    assert_keep(keep, ref["mass"], w, s, k, exact, what)
    # the GPU selection is exact on the GPU's own masses
    assert np.array_equal(keep, oracle.select(mass.astype(np.float64), w, s, k)), what
    return lse, mass, keep, ref


def test_workload1_tiny():
    wl = kvp_inputs.workload(1)
    li = kvp_inputs.make_layer(wl)
    _, _, keep, _ = full_check(li, wl.window, wl.n_sink, wl.top_k, "tiny")
    assert keep.shape == (1, 1, 52)


def test_workload2_gqa4k_full():
    wl = kvp_inputs.workload(2)
    li = kvp_inputs.make_layer(wl)
    full_check(li, wl.window, wl.n_sink, wl.top_k, "gqa4k")


@pytest.mark.parametrize("B,Hq,Hkv,S,D,w,s,k,dtype", [
    (1, 1, 1, 1, 64, 0, 0, 1, "bf16"),           # one token
    (1, 2, 1, 33, 128, 0, 4, 5, "bf16"),          # ragged, H2O case (w = 0)
    (2, 4, 2, 1000, 128, 16, 4, 64, "bf16"),      # ragged S, batch 2
    (1, 8, 1, 4097, 128, 128, 4, 512, "bf16"),    # G = 8, S = 4096 + 1
    (1, 4, 4, 700, 64, 7, 0, 100, "bf16"),        # G = 1, d = 64, no sinks
    (1, 4, 1, 300, 64, 300, 4, 8, "bf16"),        # w = S: everything is window
    (1, 4, 1, 300, 128, 400, 4, 8, "bf16"),       # w > S
    (1, 2, 1, 300, 128, 20, 4, 10000, "bf16"),    # k >= |eligible|
    (1, 2, 2, 513, 128, 1, 600, 8, "bf16"),       # sinks beyond S - w
    (3, 6, 3, 257, 128, 5, 4, 30, "f32"),         # fp32 input, exact fp32 path
    (1, 4, 2, 2048, 64, 64, 4, 256, "f32"),
])
def test_edge_shapes(B, Hq, Hkv, S, D, w, s, k, dtype):
    wl = kvp_inputs.workload(2).with_(B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, window=w, n_sink=s, top_k=k,
                                      dtype=dtype, seed=777 + S)
    li = kvp_inputs.make_layer(wl)
    full_check(li, w, s, k, f"edge S={S}")


def test_scale_override():
    wl = kvp_inputs.workload(2).with_(Hq=4, Hkv=2, S=640, seed=5)
    li = kvp_inputs.make_layer(wl)
    full_check(li, 32, 4, 50, "scale=0.05", scale=0.05)


def test_uniform_queries_closed_form():
    """Q = 0: LSE_i = ln(i+1) and mass[j] = G (H_S - H_{j+w})."""
    wl = kvp_inputs.workload(2).with_(Hq=4, Hkv=1, S=2000, seed=11)
    li = kvp_inputs.make_layer(wl, zero_q=True)
    say("[parity] uniform queries S=2000")
    lse, mass, keep = run_gpu(li, 100, 4, 64)
    S = 2000
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, S + 1)), atol=LSE_ATOL)
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, S + 1))])
    exp = np.array([4 * (H[S] - H[j + 100]) if j + 100 < S else 0.0 for j in range(S)])
    assert np.all(np.abs(mass[0, 0] - exp) <= MASS_ATOL + MASS_RTOL * exp)
    assert keep[0, 0].tolist() == list(range(68)) + list(range(S - 100, S))


def test_lse_overflow_fallback():
    """Rows whose logits exceed the first key block's maximum by more than the
    fp32 range are recomputed exactly (a key far later with a huge logit)."""
    S, D = 300, 128
    q = np.ones((1, 1, S, D), np.float32)
    k = np.random.default_rng(1).standard_normal((1, 1, S, D)).astype(np.float32) * 0.01
    k[0, 0, 200] = 13.0   # logit ~ 13*128/sqrt(128) = 147 for every query i >= 200
    say("[parity] lse fallback")
    li = kvp_inputs.LayerInputs(kvp_inputs.workload(1).with_(S=S, D=D), 0, q, k)
    lse, mass, keep = run_gpu(li, 3, 4, 10)
    ref = oracle.future_mass(q, k, 3)
    assert_lse(lse, ref["lse"], "fallback")
    assert_mass(mass, ref["mass"], "fallback")
    assert 200 in keep[0, 0].tolist()


def test_select_exact_with_ties():
    """The GPU selection against the oracle's full sort on the same fp32
    masses: bit-exact, including many exact ties."""
    rng = np.random.default_rng(3)
    for S, w, s, k in [(5000, 100, 4, 700), (4096, 128, 4, 512), (1, 0, 0, 1), (777, 0, 0, 776),
                       (131072, 1024, 4, 2048), (32768, 512, 4, 16384)]:
        say(f"[parity] select S={S} w={w} s={s} k={k}")
        m = (np.round(rng.random((3, 2, S)) * 64) / 64).astype(np.float32)
        m[0, 0] = rng.random(S).astype(np.float32) * 1e-3   # distinct small values
        keep = kvp.select_topk(torch.from_numpy(m).cuda(), w, s, k).cpu().numpy()
        ref = oracle.select(m.astype(np.float64), w, s, k)
        assert np.array_equal(keep, ref)


def test_select_row_lengths_and_alignment():
    """Every row-length path of the selection (8, 16 or 32 scores per thread
    up to 32768, the long-row kernel beyond), on both sides of each bound, with
    rows that are or are not 16-byte aligned, mixed-sign scores with ties,
    and more rows than compute units: bit-exact against the oracle's sort."""
    rng = np.random.default_rng(17)
    for S in (8192, 8193, 16384, 16385, 32767, 32768, 32769):
        w, s, k = 64, 4, S // 3
        rows = 3
        m = (np.round(rng.standard_normal((rows, S)) * 8) / 8).astype(np.float32)  # signed, with ties
        ref = oracle.select(m.reshape(rows, 1, S).astype(np.float64), w, s, k)
        for offset in (0, 1):  # offset 1: the rows start 4 bytes past a 16-byte boundary
            say(f"[parity] select rows S={S} offset={offset}")
            buf = torch.zeros(rows * S + offset, dtype=torch.float32, device="cuda")
            buf[offset:] = torch.from_numpy(m.reshape(-1)).cuda()
            dev = buf[offset:].view(rows, 1, S)
            keep = kvp.select_topk(dev, w, s, k).cpu().numpy()
            assert np.array_equal(keep, ref), (S, offset)
    # 300 rows (more than one round of workgroups), rank-like scores
    S, w, s, k = 4096, 128, 4, 1000
    m = (rng.random((300, 1, S)) ** 8 * 50).astype(np.float32)
    say("[parity] select 300 rows S=4096")
    keep = kvp.select_topk(torch.from_numpy(m).cuda(), w, s, k).cpu().numpy()
    assert np.array_equal(keep, oracle.select(m.astype(np.float64), w, s, k))


def test_select_zero_and_denormal_masses():
    S = 3000
    m = np.zeros((1, 1, S), np.float32)
    m[0, 0, 1000:1010] = np.float32(1e-42)  # subnormal
    m[0, 0, 2000] = 5.0
    keep = kvp.select_topk(torch.from_numpy(m).cuda(), 10, 4, 20).cpu().numpy()
    assert np.array_equal(keep, oracle.select(m.astype(np.float64), 10, 4, 20))


def test_deterministic():
    wl = kvp_inputs.workload(2).with_(S=3000, seed=9)
    li = kvp_inputs.make_layer(wl)
    say("[parity] determinism")
    a = run_gpu(li, 64, 4, 200)
    b = run_gpu(li, 64, 4, 200)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                              y.view(np.uint32) if y.dtype == np.float32 else y)


def test_split_group_sums_deterministic_and_equal_to_head_sums():
    """Short sequences split each group's heads over two workgroups that add
    into the zeroed output: two terms, so repeated runs are bitwise equal,
    and the result is the sum of the per-head masses up to fp32 rounding."""
    import torch
    import future_attention_scoring_kvp_amd as kvp
    wl = kvp_inputs.workload(2).with_(S=2000, seed=21)  # 8 KV heads x 8 tiles: a small grid
    li = kvp_inputs.make_layer(wl)
    say("[parity] split group sums")
    q, k = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, k)
    runs = [kvp.future_mass(q, k, lse, 64) for _ in range(3)]
    mh = kvp.future_mass_per_head(q, k, lse, 64)
    torch.cuda.synchronize()
    for r in runs[1:]:
        assert torch.equal(r.view(torch.int32), runs[0].view(torch.int32))
    G = wl.Hq // wl.Hkv
    ref = mh.view(1, wl.Hkv, G, wl.S).double().sum(2)
    assert ((runs[0].double() - ref).abs() <= 1e-6 + 1e-5 * ref.abs()).all()


def test_empty_inputs():
    q = torch.empty(1, 4, 0, 128, dtype=torch.bfloat16, device="cuda")
    lse = kvp.lse_fwd(q, q[:, :2])
    mass = kvp.future_mass(q, q[:, :2], lse, 4)
    keep = kvp.select_topk(mass, 4, 4, 8)
    assert lse.shape == (1, 4, 0) and mass.shape == (1, 2, 0) and keep.shape == (1, 2, 0)
    q0 = torch.empty(0, 4, 16, 128, dtype=torch.bfloat16, device="cuda")
    assert kvp.lse_fwd(q0, q0[:, :2]).shape == (0, 4, 16)


def test_side_stream():
    wl = kvp_inputs.workload(2).with_(Hq=8, Hkv=2, S=1500, seed=21)
    li = kvp_inputs.make_layer(wl)
    say("[parity] side stream")
    st = torch.cuda.Stream()
    q, k = to_dev(li.q), to_dev(li.k)
    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        lse = kvp.lse_fwd(q, k)
        mass = kvp.future_mass(q, k, lse, 50)
    st.synchronize()
    ref = oracle.future_mass(li.q, li.k, 50)
    assert_mass(mass.cpu().numpy(), ref["mass"], "side stream")
