"""bench.py's host-side contract, checked without a GPU: the one-GPU rule,
the kernel-source hash and the lookup of the recorded HBM traffic."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_sha_flag_prints_the_mass_kernel_hash():
    r = run_bench("--sha")
    assert r.returncode == 0
    assert re.fullmatch(r"[0-9a-f]{64}\n", r.stdout)
    assert r.stdout.strip() == bench.mass_sources_sha256()


def test_recorded_traffic_lookup(tmp_path, monkeypatch):
    summary = tmp_path / "summary.md"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", "summary.md")
    # sources are hashed from the real tree
    monkeypatch.setattr(bench, "MASS_SOURCES", tuple(os.path.join(ROOT, p) for p in bench.MASS_SOURCES))
    assert bench.recorded_traffic("w") is None                      # no summary
    sha = bench.mass_sources_sha256()
    summary.write_text(f"text\nworkload: w\nkernel_sources_sha256: {sha}\n"
                       "traffic_bytes_per_launch: 12345\n")
    assert bench.recorded_traffic("w") == 12345
    assert bench.recorded_traffic("other") is None                  # another workload
    summary.write_text(f"workload: w\nkernel_sources_sha256: {'0' * 64}\n"
                       "traffic_bytes_per_launch: 12345\n")
    assert bench.recorded_traffic("w") is None                      # the kernel changed since


def test_mass_pairs_counts_the_future_triangle():
    # S = 4, w = 1: keys 0..2 have 3, 2, 1 future queries, key 3 none
    assert bench.mass_pairs(1, 1, 4, 1) == 6
    assert bench.mass_pairs(2, 3, 4, 1) == 36
    assert bench.mass_pairs(1, 1, 4, 4) == 0
    assert bench.mass_pairs(1, 1, 4, 9) == 0


def test_cpu_baseline_sample_is_bounded():
    import kvp_inputs
    wl = kvp_inputs.workload(1)                      # S = 256, w = 16, one head
    li = kvp_inputs.make_layer(wl, 0)
    full = bench.mass_pairs(1, 1, wl.S, wl.window)
    whole = bench.cpu_baseline(wl, li, 1)
    assert whole["kind"] == "oracle" and whole["value"] > 0
    assert f"all {wl.S} query rows: {full} future-mass pairs" in whole["sample"]
    part = bench.cpu_baseline(wl, li, 1, max_pairs=full / 4)
    m = re.search(r"the last (\d+) of 256 query rows: (\d+) future-mass pairs", part["sample"])
    assert m, part["sample"]
    rows, pairs = int(m.group(1)), int(m.group(2))
    # the pairs of the last `rows` rows, and the largest such count within the bound
    tail = sum(i - wl.window + 1 for i in range(wl.S - rows, wl.S) if i >= wl.window)
    assert pairs == tail <= full / 4
    assert tail + (wl.S - rows - 1 - wl.window + 1) > full / 4


def test_cpu_baseline_parity_leg_and_single_thread():
    """The parity leg against the oracle's own values is ok; a perturbed mass
    is counted; small samples are also timed on one thread."""
    import numpy as np
    import kvp_inputs
    import oracle
    wl = kvp_inputs.workload(1)
    li = kvp_inputs.make_layer(wl, 0)
    ref = oracle.future_mass(li.q, li.k, wl.window, f32_exact=True)
    keep = oracle.select(ref["mass"], wl.window, wl.n_sink, wl.top_k)
    gpu = (ref["lse"].astype(np.float32), ref["mass"].astype(np.float32), keep)
    out = bench.cpu_baseline(wl, li, 1, gpu=gpu)
    p = out["parity"]
    assert p["ok"] and p["keep"] == ["exact"] and p["mass_violations"] == 0
    assert p["lse_max_abs_err"] < 1e-6
    assert out["single_thread"]["cores"] == 1 and out["single_thread"]["value"] > 0
    bad = ref["mass"].astype(np.float32).copy()
    bad[0, 0, 7] *= 1.01
    out = bench.cpu_baseline(wl, li, 1, gpu=(gpu[0], bad, keep))
    assert not out["parity"]["ok"] and out["parity"]["mass_violations"] == 1


def test_keep_status_rules():
    import numpy as np
    S, w, s, k = 20, 2, 2, 4
    mass = np.linspace(1.0, 0.1, S)            # strictly decreasing: the top-k are 2..5
    exact = np.array(sorted(set(range(s)) | set(range(S - w, S)) | {2, 3, 4, 5}))
    assert bench.keep_status(exact, mass, S, w, s, k, exact) == "exact"
    other = np.array(sorted(set(range(s)) | set(range(S - w, S)) | {2, 3, 4, 6}))
    assert bench.keep_status(other, mass, S, w, s, k, exact) == "differs"
    tied = mass.copy()
    tied[5] = tied[6] = 0.7                    # the k-th and (k+1)-th tie
    ex2 = np.array(sorted(set(range(s)) | set(range(S - w, S)) | {2, 3, 4, 5}))
    alt = np.array(sorted(set(range(s)) | set(range(S - w, S)) | {2, 3, 4, 6}))
    assert bench.keep_status(alt, tied, S, w, s, k, ex2) == "tie-band"
