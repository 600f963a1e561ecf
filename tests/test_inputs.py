"""Seeded input generator: determinism, distribution, recipe structure."""
import numpy as np
import torch

import kvp_inputs as gen


def test_normals_deterministic_and_counter_based():
    key = gen.stream_key(123, gen.TAG_Q)
    a = gen.normals(key, 1000)
    b = gen.normals(key, 1000)
    np.testing.assert_array_equal(a, b)
    # element n is independent of how the range is split
    c = np.concatenate([gen.normals(key, 333), gen.normals(key, 667, offset=333)])
    np.testing.assert_array_equal(a, c)
    assert not np.array_equal(a, gen.normals(gen.stream_key(124, gen.TAG_Q), 1000))


def test_normals_distribution():
    z = gen.normals(gen.stream_key(5, 1), 400000)
    assert abs(z.mean()) < 0.01
    assert abs(z.std() - 1.0) < 0.01
    # tails roughly Gaussian: P(|z| > 2) ~ 0.0455
    assert abs(np.mean(np.abs(z) > 2) - 0.0455) < 0.003


def test_tensor_thread_independent_and_bf16_rne():
    wl = gen.workload(2).with_(S=300, Hq=4, Hkv=2)
    a = gen.make_layer(wl, nthreads=1)
    b = gen.make_layer(wl, nthreads=7)
    np.testing.assert_array_equal(a.q, b.q)
    np.testing.assert_array_equal(a.k, b.k)
    f = gen.make_layer(wl.with_(dtype="f32"))
    rne = torch.from_numpy(f.k).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(rne, a.k)


def test_heavy_hitters_and_sink():
    wl = gen.workload(2).with_(S=1000, Hq=4, Hkv=2, D=64)
    li = gen.make_layer(wl)
    assert len(li.heavy) == 10 and len(set(li.heavy.tolist())) == 10
    assert li.heavy.min() >= 1 and li.heavy.max() < 1000
    base = gen.make_layer(wl.with_(sink_scale=1.0, heavy_frac=0.0))
    k, k0 = li.k_f32(), base.k_f32()
    # K row 0 x4, heavy rows x3 (in every KV head), others unchanged
    np.testing.assert_allclose(k[:, :, 0], 4 * k0[:, :, 0], rtol=1e-2, atol=1e-6)
    np.testing.assert_allclose(k[:, :, li.heavy], 3 * k0[:, :, li.heavy], rtol=1e-2, atol=1e-6)
    rest = np.setdiff1d(np.arange(1, 1000), li.heavy)
    np.testing.assert_array_equal(k[:, :, rest], k0[:, :, rest])
    np.testing.assert_array_equal(li.q, base.q)


def test_lowrank_component_concentrates_attention():
    wl = gen.workload(3).with_(B=1, S=512, Hq=4, Hkv=2)
    li = gen.make_layer(wl)
    flat = gen.make_layer(wl.with_(lowrank_rank=0, lowrank_scale=0.0))
    q, k = li.q_f32().astype(np.float64), li.k_f32().astype(np.float64)
    qf, kf = flat.q_f32().astype(np.float64), flat.k_f32().astype(np.float64)
    L = q[0, 0] @ k[0, 0].T / np.sqrt(128)
    Lf = qf[0, 0] @ kf[0, 0].T / np.sqrt(128)
    assert L.std() > 2.0 * Lf.std()   # adds ~2.8 a_i.a_j to the logits


def test_workload_table():
    assert gen.workload(1).dtype == "f32" and gen.workload(1).S == 256
    w4 = gen.workload(4)
    assert (w4.layers, w4.S, w4.Hq, w4.Hkv, w4.window, w4.top_k) == (36, 32768, 32, 8, 512, 16384)
    w5 = gen.workload(5)
    assert (w5.Hq // w5.Hkv, w5.S, w5.window, w5.top_k) == (8, 131072, 1024, 2048)
    assert w4.layer_seed(3) == 20261202 + 4000 + 3


def test_zero_q():
    li = gen.make_layer(gen.workload(1), zero_q=True)
    assert li.q.dtype == np.float32 and not li.q.any()
