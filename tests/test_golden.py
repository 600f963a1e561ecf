"""Stored fixtures under tests/golden/: the pages' printed budget example and
a snapshot of the oracle on one small seeded input."""
import json
import os

import numpy as np

import kvp_inputs
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_kvpop_budget_compression_ratio():
    """KVpop §4.1: budgets 2048 / 4096 at S = 16384 are 88% / 75% compression.
    The keep-set of every split s + w + k = B (§3 Eq. 1) has exactly B tokens
    when S >= B."""
    fx = json.load(open(os.path.join(GOLDEN, "kvpop_budget_compression.json")))
    S = fx["seq_len"]
    for case in fx["cases"]:
        B = case["budget"]
        for s, w in ((4, 128), (16, 512), (0, 1024)):
            n_keep = oracle.keep_count(S, w, s, B - s - w)
            assert n_keep == B
            assert round(100 * (1 - n_keep / S)) == case["compression_pct"]


def test_oracle_snapshot_unchanged():
    fx = json.load(open(os.path.join(GOLDEN, "oracle_snapshot_s96.json")))
    wl = kvp_inputs.workload(1).with_(S=fx["S"], window=fx["window"], n_sink=fx["n_sink"],
                                      top_k=fx["top_k"])
    li = kvp_inputs.make_layer(wl)
    out = oracle.future_mass(li.q, li.k, wl.window)
    np.testing.assert_allclose(out["lse"][0, 0], fx["lse"], rtol=1e-12)
    np.testing.assert_allclose(out["mass"][0, 0], fx["mass"], rtol=1e-12, atol=1e-300)
    keep = oracle.select(out["mass"], wl.window, wl.n_sink, wl.top_k)
    assert keep[0, 0].tolist() == fx["keep"]
