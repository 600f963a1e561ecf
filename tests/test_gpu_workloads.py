"""GPU parity at the full sizes of the three large workloads, in the launch
configuration the benchmark times.  The oracle runs one whole (batch, KV
head) unit of the 16K and 32K shapes here; for the 128K shape a whole KV head
is compared with oracle values stored by a committed script (minutes of CPU
work), and the tail rows of another head with the oracle run here.  Also: LSE
of sampled rows of every head, and properties that hold at any size (w = 0
total mass G*S, zero mass inside the window, exact selection on the GPU's own
masses)."""
import hashlib
import os

import numpy as np
import pytest
import torch

import future_attention_scoring_kvp_amd as kvp
import kvp_inputs
import oracle
from parity import assert_keep, assert_lse, assert_mass, say, to_dev

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def gpu_path(q, k, w, s, kk):
    lse = kvp.lse_fwd(q, k)
    mass = kvp.future_mass(q, k, lse, w)
    keep = kvp.select_topk(mass, w, s, kk)
    torch.cuda.synchronize()
    return lse, mass, keep


def sampled_rows(rng, B, Hq, S, n):
    return np.stack([rng.integers(0, B, n), rng.integers(0, Hq, n), rng.integers(0, S, n)], 1)


def common_properties(li, lse, mass, keep, q, k, what):
    wl = li.wl
    S, w, G = wl.S, wl.window, wl.G
    m = mass.cpu().numpy()
    assert np.all(np.isfinite(m)) and np.all(m >= 0), what
    assert np.all(m[:, :, S - w:] == 0), f"{what}: mass inside the window must be 0"
    kp = keep.cpu().numpy()
    assert kp.shape[-1] == kvp.keep_count(S, w, wl.n_sink, wl.top_k)
    assert np.array_equal(kp, oracle.select(m.astype(np.float64), w, wl.n_sink, wl.top_k)), \
        f"{what}: selection not exact on the GPU masses"
    # LSE of sampled rows of every head
    rng = np.random.default_rng(17)
    rows = sampled_rows(rng, wl.B, wl.Hq, S, 96)
    rows[:8, 2] = S - 1 - np.arange(8)   # include the longest rows
    ref = oracle.lse_rows(li.q, li.k, rows)
    got = lse.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert np.abs(got - ref).max() <= 1e-4, f"{what}: sampled LSE err {np.abs(got - ref).max():.3g}"
    # w = 0: every softmax row sums to one, so each KV head's total is G * S
    m0 = kvp.future_mass(q, k, lse, 0).double().sum(dim=2).cpu().numpy()
    np.testing.assert_allclose(m0, G * S, rtol=1e-4)


def test_workload3_llama8b_16k():
    wl = kvp_inputs.workload(3)
    say("[workload] llama8b_16k: generating inputs")
    li = kvp_inputs.make_layer(wl)
    q, k = to_dev(li.q), to_dev(li.k)
    say("[workload] llama8b_16k: GPU path")
    lse, mass, keep = gpu_path(q, k, wl.window, wl.n_sink, wl.top_k)
    common_properties(li, lse, mass, keep, q, k, "llama8b_16k")
    b, h = 3, 5
    say(f"[workload] llama8b_16k: oracle unit (b={b}, h={h})")
    ref = oracle.future_mass(li.q, li.k, wl.window, b_only=b, h_only=h)
    g0 = h * wl.G
    assert_lse(lse.cpu().numpy()[b, g0:g0 + wl.G], ref["lse"][b, g0:g0 + wl.G], "llama8b_16k")
    assert_mass(mass.cpu().numpy()[b, h], ref["mass"][b, h], "llama8b_16k")
    exact = oracle.select(ref["mass"][b:b + 1, h:h + 1], wl.window, wl.n_sink, wl.top_k)
    assert_keep(keep.cpu().numpy()[b:b + 1, h:h + 1], ref["mass"][b:b + 1, h:h + 1], wl.window,
                wl.n_sink, wl.top_k, exact, "llama8b_16k")


@pytest.mark.parametrize("layer,h", [(0, 0), (35, 7)])
def test_workload4_qwen3_layer(layer, h):
    wl = kvp_inputs.workload(4)
    say(f"[workload] qwen3 layer {layer}: generating inputs")
    li = kvp_inputs.make_layer(wl, layer=layer)
    q, k = to_dev(li.q), to_dev(li.k)
    say(f"[workload] qwen3 layer {layer}: GPU path")
    lse, mass, keep = gpu_path(q, k, wl.window, wl.n_sink, wl.top_k)
    common_properties(li, lse, mass, keep, q, k, f"qwen3 layer {layer}")
    say(f"[workload] qwen3 layer {layer}: oracle unit h={h}")
    ref = oracle.future_mass(li.q, li.k, wl.window, b_only=0, h_only=h)
    g0 = h * wl.G
    assert_lse(lse.cpu().numpy()[0, g0:g0 + wl.G], ref["lse"][0, g0:g0 + wl.G], "qwen3")
    assert_mass(mass.cpu().numpy()[0, h], ref["mass"][0, h], "qwen3")
    exact = oracle.select(ref["mass"][:, h:h + 1], wl.window, wl.n_sink, wl.top_k)
    assert_keep(keep.cpu().numpy()[:, h:h + 1], ref["mass"][:, h:h + 1], wl.window, wl.n_sink,
                wl.top_k, exact, "qwen3")


def test_workload5_llama70b_128k():
    """Whole KV head 3 (its 8 query heads, every one of the 131072 query rows
    and keys) against the oracle's fp64 values stored by
    tests/golden/make_config5_head.py; the tail rows of a second head against
    the oracle run here."""
    wl = kvp_inputs.workload(5)
    say("[workload] llama70b_128k: generating inputs")
    li = kvp_inputs.make_layer(wl)
    gold = np.load(os.path.join(GOLDEN, "config5_head3.npz"), allow_pickle=False)
    h = int(gold["head"])
    g0 = h * wl.G
    qh = np.ascontiguousarray(li.q[0, g0:g0 + wl.G])
    kh = np.ascontiguousarray(li.k[0, h])
    assert hashlib.sha256(qh.tobytes()).hexdigest() == str(gold["q_sha256"]) and \
        hashlib.sha256(kh.tobytes()).hexdigest() == str(gold["k_sha256"]), \
        "inputs differ from those of the stored oracle values"
    q, k = to_dev(li.q), to_dev(li.k)
    say("[workload] llama70b_128k: GPU path")
    lse, mass, keep = gpu_path(q, k, wl.window, wl.n_sink, wl.top_k)
    common_properties(li, lse, mass, keep, q, k, "llama70b_128k")
    S, w = wl.S, wl.window
    say(f"[workload] llama70b_128k: whole head {h} against the stored oracle values")
    assert_lse(lse.cpu().numpy()[0, g0:g0 + wl.G], gold["lse"].astype(np.float64),
               "llama70b_128k head LSE")
    ref_mass = gold["mass"]
    assert ref_mass.shape == (S,)
    got = mass.cpu().numpy()[0, h].astype(np.float64)
    nz = ref_mass > 0
    say(f"[workload] llama70b_128k head {h}: max rel mass err "
        f"{(np.abs(got[nz] - ref_mass[nz]) / ref_mass[nz]).max():.2e}, keep-set "
        f"{'identical' if np.array_equal(keep.cpu().numpy()[0, h], gold['keep']) else 'differs'}")
    assert_mass(mass.cpu().numpy()[0, h], ref_mass, "llama70b_128k head mass")
    assert_keep(keep.cpu().numpy()[:, h:h + 1], ref_mass.reshape(1, 1, S), w, wl.n_sink,
                wl.top_k, gold["keep"].reshape(1, 1, -1), "llama70b_128k head keep-set")

    row_lo = S - 1536
    h2 = 6
    say(f"[workload] llama70b_128k: oracle tail rows >= {row_lo} of h={h2}")
    ref = oracle.future_mass(li.q, li.k, w, b_only=0, h_only=h2, row_lo=row_lo)
    g2 = h2 * wl.G
    assert_lse(lse.cpu().numpy()[0, g2:g2 + wl.G, row_lo:], ref["lse"][0, g2:g2 + wl.G, row_lo:],
               "llama70b_128k tail")
    lo = row_lo - w   # masses of keys >= row_lo - w are complete
    assert_mass(mass.cpu().numpy()[0, h2, lo:], ref["mass"][0, h2, lo:], "llama70b_128k tail")
