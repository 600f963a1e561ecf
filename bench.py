"""Benchmark of the future-attention-mass path on one MI355X.

One step = the whole path over one batch of synthetic input: for every layer
of the workload, the causal LSE pass and the transposed future-mass pass, then
one keep-set selection over all (layer, batch, KV head) rows.  Inputs are
generated on the host from seeded recipes, uploaded once and resident in HBM
before the timed region starts.

The default workload is the Qwen3-4B-shaped stack: 36 layers, 32 query / 8 KV
heads, d = 128, batch 1, S = 32768, w = 512, 4 sinks, k = 16384.

Prints ONE JSON line on stdout (everything else goes to stderr):
  value        future-mass query-key pairs per second over whole steps
               (pairs = B * Hq * L * (S - w)(S - w + 1) / 2 per step)
  roofline     the mass kernel alone: algorithmic flops (2 d per pair) per
               launch over its average launch time, measured with HIP events
               on the stream it runs on, against the bf16 dense MFMA peak
  cpu_baseline the fp64 CPU oracle on a bounded sample of the same workload
               (with the parity of the GPU's layer 0 on that sample: LSE and
               mass errors, keep-set status)
  mfma_probe   the sustained bf16 matrix-core rate of this GPU (a pure-MFMA
               kernel) and its core clock under that load; roofline also
               states the mass kernel against that measured peak
  next_rows    after the timed steps: the per-head mass pass, the KVpop target
               epilogue, its static priorities, the running top-k cutoff over
               them, the sparse LSE, the Soft-TopK and the Golden-Eviction
               block / future scores on the same layers
  roofline.traffic is the HBM bytes per mass-kernel launch from the committed
  counter summary (profiles/), reported only while the kernel sources still
  hash to the value recorded there

    python bench.py [--steps K] [--warmup W] [--workload N] [--no-cpu-baseline]
                    [--batch B] [--hq H] [--hkv H] [--seq S] [--dim D]
                    [--window W] [--sinks N] [--topk K] [--seed N]
    python bench.py --copy-probe BYTES   # plain copy kernel, for counter scaling
    python bench.py --read-probe BYTES   # 16-byte buffer-load reads, for counter scaling
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X bf16 dense matrix peak: 256 CUs x 4 SIMDs x 1024 flop/clk x 2.4 GHz.
PEAK_BF16_TFLOPS = 2516.58
PEAK_HBM_GBS = 8000.0


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def mass_pairs(B: int, Hq: int, S: int, w: int) -> int:
    """Query-key pairs of the future-mass pass of one layer: every (query
    head, query i, key j) with j + w <= i."""
    n = max(S - w, 0)
    return B * Hq * n * (n + 1) // 2


MASS_SOURCES = ("future_attention_scoring_kvp_amd/csrc/mass_kernel.hip",
                "future_attention_scoring_kvp_amd/csrc/kvp_device.h")
TRAFFIC_SUMMARY = "profiles/mass_kernel_qwen3_4b_32k_pmc.md"


def mass_sources_sha256() -> str:
    h = hashlib.sha256()
    for rel in MASS_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload_name: str):
    """HBM bytes per mass-kernel launch recorded in the counter summary, or
    None if there is none for this workload or the kernel has changed since."""
    path = os.path.join(ROOT, TRAFFIC_SUMMARY)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    fields = dict(re.findall(r"^([a-z_0-9]+):\s*(\S+)\s*$", text, flags=re.M))
    if fields.get("workload") != workload_name:
        return None
    if fields.get("kernel_sources_sha256") != mass_sources_sha256():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_probe(nbytes: int, reps: int) -> None:
    import torch
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    log(f"copy probe: {reps} copies of {nbytes} bytes")
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}))


def read_probe(nbytes: int, reps: int) -> None:
    """The 16-byte buffer-load read probe (libkvp_probe.so) over `nbytes`
    bytes, `reps` launches: the counter reading of a known read through the
    kernels' own load instruction."""
    import ctypes
    import torch
    import future_attention_scoring_kvp_amd as kvp
    lib = ctypes.CDLL(os.path.join(os.path.dirname(kvp.library_path()), "libkvp_probe.so"))
    lib.kvp_probe_read16.restype = ctypes.c_int
    lib.kvp_probe_read16.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p]
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    blocks = 4096
    sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    for _ in range(reps):
        rc = lib.kvp_probe_read16(src.data_ptr(), nbytes, blocks, sink.data_ptr(),
                                  int(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"read probe failed ({rc})")
    torch.cuda.synchronize()
    log(f"read probe: {reps} reads of {nbytes} bytes through 16-byte buffer loads")
    print(json.dumps({"read_probe_bytes": nbytes, "reps": reps}))


def cpu_baseline(wl, li0, n_heads: int, gpu=None, max_pairs: float = 4.5e9,
                 single_thread_pairs: float = 2e8) -> dict:
    """The CPU oracle (dense fp64 softmax rows + explicit column sums), as it
    stands, on whole (batch 0, KV head) units 0 .. n_heads-1 of layer 0: the
    query rows of their G query heads from row_lo on, row_lo = 0 unless that
    would exceed max_pairs future-mass pairs (long sequences: the last rows,
    each computed in full).  Returns the future-mass pairs per second the
    sample covers (its LSE work included in the time).  With ``gpu`` = the
    GPU's layer-0 (lse [B,Hq,S], mass [B,Hkv,S], keep [B,Hkv,n]) as numpy
    arrays, also the parity of the sample: LSE of its rows, masses of the keys
    its rows complete, and (whole units only) the keep-sets.  Samples of at
    most single_thread_pairs pairs are timed on one thread as well."""
    import numpy as np
    import oracle
    S, w, G = wl.S, wl.window, wl.G
    n_heads = max(1, min(n_heads, wl.Hkv))

    def pairs_from(row_lo):  # future-mass pairs of rows >= row_lo: keys j <= i - w
        lo = max(row_lo, w)
        n = S - w
        return n_heads * G * (n * (n + 1) // 2 - (lo - w) * (lo - w + 1) // 2) if lo < S else 0

    row_lo = 0
    if pairs_from(0) > max_pairs:
        lo, hi = 0, S
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if pairs_from(mid) > max_pairs:
                lo = mid
            else:
                hi = mid
        row_lo = hi
    threads = oracle.default_threads()
    refs = []
    t0 = time.perf_counter()
    for h in range(n_heads):
        refs.append(oracle.future_mass(li0.q, li0.k, w, b_only=0, h_only=h, row_lo=row_lo,
                                       nthreads=threads, f32_exact=wl.dtype == "f32"))
    dt = time.perf_counter() - t0
    pairs = pairs_from(row_lo)
    rows = "all" if row_lo == 0 else f"the last {S - row_lo} of"
    out = {"value": pairs / dt / 1e9, "unit": "G query-key pairs/s", "cores": threads,
           "kind": "oracle", "seconds": round(dt, 3),
           "sample": (f"layer 0, batch 0, KV heads 0..{n_heads - 1} ({n_heads * G} query heads), "
                      f"{rows} {S} query rows: {pairs} future-mass pairs, LSE included")}
    if pairs <= single_thread_pairs and threads > 1:
        # small samples (the tiny and 4K workloads) are also timed on one thread
        t1 = time.perf_counter()
        for h in range(n_heads):
            oracle.future_mass(li0.q, li0.k, w, b_only=0, h_only=h, row_lo=row_lo, nthreads=1,
                               f32_exact=wl.dtype == "f32")
        d1 = time.perf_counter() - t1
        out["single_thread"] = {"value": pairs / d1 / 1e9, "cores": 1, "seconds": round(d1, 3)}
    if gpu is not None:
        lse_g, mass_g, keep_g = gpu
        lse_err, rel_err, n_bad, statuses = 0.0, 0.0, 0, []
        key_lo = max(0, row_lo - w)  # keys whose every future row is in the sample
        for h, ref in enumerate(refs):
            g0 = h * G
            d = np.abs(lse_g[0, g0:g0 + G, row_lo:] - ref["lse"][0, g0:g0 + G, row_lo:])
            lse_err = max(lse_err, float(d.max()))
            o = ref["mass"][0, h, key_lo:]
            g = mass_g[0, h, key_lo:].astype(np.float64)
            n_bad += int((np.abs(g - o) > 1e-5 + 2e-3 * np.abs(o)).sum())
            nz = o > 0
            if nz.any():
                rel_err = max(rel_err, float((np.abs(g[nz] - o[nz]) / o[nz]).max()))
            if row_lo == 0:
                m = ref["mass"][:, h:h + 1]
                exact = oracle.select(m, w, wl.n_sink, wl.top_k)[0, 0]
                statuses.append(keep_status(keep_g[0, h], m[0, 0], S, w, wl.n_sink, wl.top_k,
                                            exact))
        out["parity"] = {
            "lse_max_abs_err": lse_err, "lse_tol": 1e-4,
            "mass_max_rel_err": rel_err, "mass_violations": n_bad,
            "mass_tol": "1e-5 + 2e-3 |oracle|", "mass_keys": f"{key_lo}..{S - 1}",
            "keep": statuses if statuses else "not compared (partial unit)",
            "ok": lse_err <= 1e-4 and n_bad == 0 and all(x != "differs" for x in statuses)}
    return out


def mfma_probe(torch, blocks: int = 256, iters: int = 20000, reps: int = 5) -> dict:
    """The matrix-core probe (libkvp_probe.so): best rate of `reps` launches
    of back-to-back bf16 MFMAs on every CU, and the mean core clock of its
    workgroups (core-clock counter over the constant-rate counter)."""
    import ctypes
    import future_attention_scoring_kvp_amd as kvp
    path = os.path.join(os.path.dirname(kvp.library_path()), "libkvp_probe.so")
    lib = ctypes.CDLL(path)
    lib.kvp_probe_mfma_bf16.restype = ctypes.c_int
    lib.kvp_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]
    lib.kvp_probe_flops.restype = ctypes.c_double
    lib.kvp_probe_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.kvp_probe_wall_clock_khz.restype = ctypes.c_int
    sink = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    stamps = torch.zeros(blocks * 4, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    best_ms, clocks = None, []
    for r in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = lib.kvp_probe_mfma_bf16(blocks, iters, sink.data_ptr(), stamps.data_ptr(),
                                     int(stream.cuda_stream))
        e1.record(stream)
        torch.cuda.synchronize()
        if rc != 0:
            raise RuntimeError(f"mfma probe failed ({rc})")
        if r == 0:
            continue  # warm-up
        ms = e0.elapsed_time(e1)
        best_ms = ms if best_ms is None else min(best_ms, ms)
        st = stamps.view(blocks, 4).cpu().double()
        clocks.append(((st[:, 1] - st[:, 0]) / (st[:, 3] - st[:, 2])).mean().item())
    khz = lib.kvp_probe_wall_clock_khz()
    tflops = lib.kvp_probe_flops(blocks, iters) / (best_ms * 1e-3) / 1e12
    ghz = sum(clocks) / len(clocks) * khz * 1e3 / 1e9 if khz > 0 else None
    log(f"bench: MFMA probe {tflops:.1f} TFLOP/s ({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of the "
        f"datasheet peak), core clock {ghz:.3f} GHz" if ghz else
        f"bench: MFMA probe {tflops:.1f} TFLOP/s")
    return {"tflops": round(tflops, 2), "clock_ghz": round(ghz, 3) if ghz else None,
            "frac_of_datasheet": round(tflops / PEAK_BF16_TFLOPS, 4),
            "kernel": f"{blocks} workgroups x 8 waves x {16 * iters} v_mfma_f32_32x32x16_bf16, "
                      f"register operands; best of {reps}"}


def graph_replay(torch, step, reps: int, pairs_step: int, outs) -> dict:
    """The same step captured once into a HIP graph and replayed: two checked
    replays (outputs cleared first, then compared bit for bit with the eager
    step's), then `reps` timed replays.  Reported beside the eager figures; the
    JSON line's value stays the eager one."""
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    equal = True
    for _ in range(2):
        for o in outs:
            o.fill_(-3 if o.dtype == torch.int32 else float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        equal &= all(torch.equal(o, r) for o, r in zip(outs, ref))
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / reps
    equal &= all(torch.equal(o, r) for o, r in zip(outs, ref))
    log(f"bench: graph replay {ms:.3f} ms per step, outputs equal to the eager step: {equal}")
    return {"ms_per_step": round(ms, 4), "gpairs_per_s": round(pairs_step / (ms * 1e-3) / 1e9, 3),
            "replays": reps, "outputs_equal_eager": bool(equal)}


def keep_status(keep, mass, S, w, s, k, exact) -> str:
    """'exact' when the GPU keep-set equals the oracle's; 'tie-band' when it
    differs only among tokens whose oracle masses lie within the mass
    tolerance of the k-th one (and the k-th and (k+1)-th are that close);
    'differs' otherwise."""
    import numpy as np
    if np.array_equal(keep, exact):
        return "exact"
    tol = lambda v: 1e-5 + 2e-3 * abs(v)  # noqa: E731
    elig = np.arange(s, S - w) if S - w > s else np.arange(0)
    kk = min(k, len(elig))
    if kk in (0, len(elig)) or len(keep) != len(exact):
        return "differs"
    order = elig[np.lexsort((elig, -mass[elig]))]
    vk, vk1 = mass[order[kk - 1]], mass[order[kk]]
    if vk - vk1 > tol(vk):
        return "differs"
    fixed = set(range(min(s, S))) | set(range(max(0, S - w), S))
    chosen = set(keep.tolist()) - fixed
    if not fixed <= set(keep.tolist()) or not chosen <= set(elig.tolist()):
        return "differs"
    above = set(elig[mass[elig] > vk + tol(vk)].tolist())
    below = set(elig[mass[elig] < vk - tol(vk)].tolist())
    return "tie-band" if above <= chosen and not (below & chosen) else "differs"


def next_rows(kvp, torch, wl, L, q_all, k_all, lse_all, stream) -> dict:
    """Per-launch times of the entry points beyond the three-stage path, on
    the same resident layers (not part of the timed steps): the per-query-head
    mass pass (every layer), the target epilogue over all layers' per-head
    masses in one launch, the running top-k cutoff over all (layer, KV head)
    rows of those scores in one launch, the sparse LSE of layer 0 under that
    cutoff, LKV's Soft-TopK forward and backward over those rows, and the
    Golden-Eviction block and future scores (every layer)."""
    B, Hq, Hkv, S, D = wl.B, wl.Hq, wl.Hkv, wl.S, wl.D
    w, s, k = wl.window, wl.n_sink, wl.top_k
    dev = q_all.device
    mh_all = torch.empty((L * B, Hq, S), dtype=torch.float32, device=dev)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def per_head_all():
        for l in range(L):
            kvp.future_mass_per_head(q_all[l], k_all[l], lse_all[l], w,
                                     out=mh_all[l * B:(l + 1) * B])

    ph_ms = timed(per_head_all, 1) / L
    pairs = mass_pairs(B, Hq, S, w)
    score = torch.empty((L * B, Hkv, S), dtype=torch.float32, device=dev)
    tgt_ms = timed(lambda: kvp.target_scores(mh_all, Hkv, w, agg=kvp.AGG_MEAN_LOG, eps=1e-6,
                                             out=score), 10)
    tgt_bytes = 4 * L * B * (Hq + Hkv) * S
    # Golden-Eviction block / future scores with ForesightKV's training budget
    # and eviction length (first 1024 rows, blocks of 256), window 0
    b_start, b_len = 1024, 256
    nb = kvp.block_count(S, b_start, b_len)
    blk_buf = fut_buf = None
    blk_ms = 0.0
    if nb > 0:
        def blocks_all():
            for l in range(L):
                kvp.block_future_scores(q_all[l], k_all[l], lse_all[l], b_start, b_len)
        blk_ms = timed(blocks_all, 1) / L
    blk_pairs = B * Hq * (S * (S + 1) // 2 - b_start * (b_start + 1) // 2) if nb > 0 else 0
    rows = L * B * Hkv
    # static priorities of the decayed target (App. B.3 leaves gamma_h and n open:
    # n = 64 and gamma_h from 0.90 to 0.99 over the KV heads), the running
    # cutoff's input
    n_decay = 64
    lg = torch.log(torch.linspace(0.90, 0.99, Hkv, dtype=torch.float32, device=dev))
    pri = torch.empty_like(score)
    pri_ms = timed(lambda: kvp.static_priority(score, n_decay, lg, out=pri), 10)
    ws = torch.empty(max(1, 20 * rows * (S - min(s, S))), dtype=torch.uint8, device=dev)
    cut_ms = timed(lambda: kvp.running_cutoff(pri, w, s, k, workspace=ws), 3)
    # the sparse normaliser of KVpop's student on layer 0, with the running
    # cutoff of its own target scores (window, sinks, budget of the workload)
    rk_all, ct_all = kvp.running_cutoff(pri, w, s, k, workspace=ws)
    sp_out = torch.empty_like(lse_all[0])
    sp_ms = timed(lambda: kvp.lse_sparse(q_all[0], k_all[0], rk_all[:B], ct_all[:B], w,
                                         out=sp_out), 3)
    lse_pairs = B * Hq * S * (S + 1) // 2
    # LKV Soft-TopK over the same rows with the same budget, forward and backward
    st_k = torch.full((rows,), float(k), dtype=torch.float32, device=dev)
    st_in = score.view(rows, S)
    st_out = {}

    def st_fwd():
        st_out["y"], st_out["lam"] = kvp.soft_topk(st_in, st_k, 1.0)

    st_fwd_ms = timed(st_fwd, 3)
    st_dy = torch.ones_like(st_in)
    st_bwd_ms = timed(lambda: kvp.soft_topk_backward(st_in, st_out["lam"], st_dy, 1.0), 3)
    log(f"bench: per-head mass {ph_ms:.3f} ms/layer, target {tgt_ms:.4f} ms, "
        f"static priority {pri_ms:.4f} ms, "
        f"running cutoff {cut_ms:.3f} ms ({rows} rows), sparse LSE {sp_ms:.3f} ms/layer, "
        f"soft top-k {st_fwd_ms:.3f} + "
        f"{st_bwd_ms:.3f} ms, block scores {blk_ms:.3f} ms/layer")
    return {
        "mass_per_head": {"ms_per_layer": round(ph_ms, 4),
                          "gpairs_per_s": round(pairs / (ph_ms * 1e-3) / 1e9, 3),
                          "frac_bf16_peak": round(pairs * 2 * D / (ph_ms * 1e-3) / 1e12
                                                  / PEAK_BF16_TFLOPS, 4)},
        "target_scores": {"ms_all_layers": round(tgt_ms, 4), "bytes": tgt_bytes,
                          "gbs": round(tgt_bytes / (tgt_ms * 1e-3) / 1e9, 1),
                          "frac_hbm": round(tgt_bytes / (tgt_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                          "agg": "mean of logs, count-normalised, eps 1e-6"},
        "static_priority": {"ms_all_layers": round(pri_ms, 4), "decay_step": n_decay,
                            "gamma": "0.90..0.99 over the KV heads",
                            "gbs": round(8 * rows * S / (pri_ms * 1e-3) / 1e9, 1)},
        "running_cutoff": {"ms_all_layers": round(cut_ms, 4), "rows": rows, "keys_per_row": S,
                           "input": "static priorities of the decayed targets",
                           "mkeys_per_s": round(rows * S / (cut_ms * 1e-3) / 1e6, 1)},
        "lse_sparse": {"ms_per_layer": round(sp_ms, 4),
                       "gpairs_per_s": round(lse_pairs / (sp_ms * 1e-3) / 1e9, 3),
                       "frac_bf16_peak": round(lse_pairs * 2 * D / (sp_ms * 1e-3) / 1e12
                                               / PEAK_BF16_TFLOPS, 4)},
        "soft_topk": {"fwd_ms_all_rows": round(st_fwd_ms, 4), "bwd_ms_all_rows": round(st_bwd_ms, 4),
                      "rows": rows, "n": S, "k": k},
        "block_future_scores": {"ms_per_layer": round(blk_ms, 4), "block_start": b_start,
                                "block_len": b_len, "blocks": nb,
                                "gpairs_per_s": round(blk_pairs / (blk_ms * 1e-3) / 1e9, 3)
                                if blk_ms > 0 else None,
                                "frac_bf16_peak": round(blk_pairs * 2 * D / (blk_ms * 1e-3) / 1e12
                                                        / PEAK_BF16_TFLOPS, 4)
                                if blk_ms > 0 else None},
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (0 = workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=2,
                    help="whole KV heads of layer 0 in the oracle sample")
    ap.add_argument("--no-extras", action="store_true", help="skip the next_rows timings")
    ap.add_argument("--no-probe", action="store_true", help="skip the MFMA peak probe")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay of the step (timed after the eager steps)")
    for name, field, what in (("batch", "B", "batch"), ("hq", "Hq", "query heads"),
                              ("hkv", "Hkv", "KV heads"), ("seq", "S", "sequence length"),
                              ("dim", "D", "head dimension"), ("window", "window", "window w"),
                              ("sinks", "n_sink", "sink tokens s"), ("topk", "top_k", "budget k"),
                              ("seed", "seed", "base seed of the input generator")):
        ap.add_argument(f"--{name}", dest=f"ov_{field}", type=int, default=None,
                        help=f"override the workload's {what}")
    ap.add_argument("--sha", action="store_true", help="print the mass kernel sources' sha256")
    ap.add_argument("--copy-probe", type=int, default=0)
    ap.add_argument("--copy-reps", type=int, default=5)
    ap.add_argument("--read-probe", type=int, default=0,
                    help="read BYTES through 16-byte buffer loads (counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the path has no multi-GPU mode "
              "(each (layer, batch, KV head) unit is independent and would shard with no "
              "exchange)", file=sys.stderr)
        return 2

    if args.sha:
        print(mass_sources_sha256())
        return 0
    import torch
    if args.copy_probe:
        copy_probe(args.copy_probe, args.copy_reps)
        return 0
    if args.read_probe:
        read_probe(args.read_probe, args.copy_reps)
        return 0

    import future_attention_scoring_kvp_amd as kvp
    import kvp_inputs

    kvp.load_library()  # fails loudly if the HIP library is not built
    wl = kvp_inputs.workload(args.workload)
    overrides = {k[3:]: v for k, v in vars(args).items() if k.startswith("ov_") and v is not None}
    if overrides:
        wl = wl.with_(**overrides)
    L = args.layers or wl.layers
    B, Hq, Hkv, S, D, G = wl.B, wl.Hq, wl.Hkv, wl.S, wl.D, wl.G
    w, s, k = wl.window, wl.n_sink, wl.top_k
    dev = torch.device("cuda:0")
    tdtype = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

    log(f"bench: workload {wl.name}, {L} layers, B={B} Hq={Hq} Hkv={Hkv} S={S} d={D} "
        f"w={w} s={s} k={k}")
    q_all = torch.empty((L, B, Hq, S, D), dtype=tdtype, device=dev)
    k_all = torch.empty((L, B, Hkv, S, D), dtype=tdtype, device=dev)
    li0 = None
    t0 = time.perf_counter()
    for l in range(L):
        li = kvp_inputs.make_layer(wl, layer=l)
        if l == 0:
            li0 = li
        for src, dst in ((li.q, q_all[l]), (li.k, k_all[l])):
            t = torch.from_numpy(src.view("int16") if src.dtype.name == "uint16" else src)
            dst.copy_(t.view(tdtype) if src.dtype.name == "uint16" else t)
        if l % 6 == 5 or l == L - 1:
            log(f"bench: generated and uploaded {l + 1}/{L} layers ({time.perf_counter() - t0:.1f} s)")
    lse_all = torch.empty((L, B, Hq, S), dtype=torch.float32, device=dev)
    mass_all = torch.empty((L, B, Hkv, S), dtype=torch.float32, device=dev)
    n_keep = kvp.keep_count(S, w, s, k)
    keep_all = torch.empty((L * B, Hkv, n_keep), dtype=torch.int32, device=dev)
    sel_ws_bytes = kvp.select_workspace_bytes(L * B * Hkv, S, k)
    sel_ws = torch.empty(sel_ws_bytes, dtype=torch.uint8, device=dev) if sel_ws_bytes else None
    # short sequences: the chunked mass launch, with its workspace allocated here
    mass_ws_bytes = kvp.future_mass_workspace_bytes(q_all[0], k_all[0], w)
    mass_ws = torch.empty(mass_ws_bytes, dtype=torch.uint8, device=dev) if mass_ws_bytes else None
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(events=None):
        for l in range(L):
            if events is not None:
                events[l][0].record(stream)
            kvp.lse_fwd(q_all[l], k_all[l], out=lse_all[l])
            if events is not None:
                events[l][1].record(stream)
            if mass_ws is not None:
                kvp.future_mass_chunked(q_all[l], k_all[l], lse_all[l], w, workspace=mass_ws,
                                        out=mass_all[l])
            else:
                kvp.future_mass(q_all[l], k_all[l], lse_all[l], w, out=mass_all[l])
            if events is not None:
                events[l][2].record(stream)
        kvp.select_topk(mass_all.view(L * B, Hkv, S), w, s, k, out=keep_all, workspace=sel_ws)
        if events is not None:
            events[L][0].record(stream)

    log(f"bench: {args.warmup} warmup steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(L + 1)]
          for _ in range(args.steps)]
    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for it in range(args.steps):
        step(ev[it])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    lse_ms = mass_ms = sel_ms = 0.0
    for it in range(args.steps):
        e = ev[it]
        for l in range(L):
            lse_ms += e[l][0].elapsed_time(e[l][1])
            mass_ms += e[l][1].elapsed_time(e[l][2])
        sel_ms += e[L - 1][2].elapsed_time(e[L][0])
    n_mass = args.steps * L
    mass_launch_ms = mass_ms / n_mass
    lse_launch_ms = lse_ms / n_mass
    sel_launch_ms = sel_ms / args.steps
    ms_per_step = wall * 1e3 / args.steps

    pairs_layer = mass_pairs(B, Hq, S, w)
    pairs_step = pairs_layer * L
    value = pairs_step / (ms_per_step * 1e-3) / 1e9
    flops_launch = pairs_layer * 2 * D
    achieved = flops_launch / (mass_launch_ms * 1e-3) / 1e12
    lse_pairs = B * Hq * S * (S + 1) // 2
    sel_bytes = 4 * L * B * Hkv * S + 4 * L * B * Hkv * n_keep
    log(f"bench: step {ms_per_step:.3f} ms; per layer LSE {lse_launch_ms:.3f} ms, mass "
        f"{mass_launch_ms:.3f} ms ({achieved:.1f} TFLOP/s, "
        f"{100 * achieved / PEAK_BF16_TFLOPS:.1f}% of bf16 peak); select {sel_launch_ms:.3f} ms")

    out = {
        "metric": "future-mass G query-key pairs/s per GPU; % of bf16 MFMA peak",
        "value": round(value, 3),
        "unit": "G query-key pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K with the workload's heavy-hitter recipe)",
        "config": {"workload": wl.name, "layers": L, "batch": B, "n_q_heads": Hq,
                   "n_kv_heads": Hkv, "seq_len": S, "head_dim": D, "window": w,
                   "n_sink": s, "top_k": k, "seed": wl.layer_seed(0),
                   "overrides": overrides or None, "parallelism": "none (1 GPU)"},
        "stages_ms": {"lse_per_layer": round(lse_launch_ms, 4),
                      "mass_per_layer": round(mass_launch_ms, 4),
                      "select_all_layers": round(sel_launch_ms, 4)},
        "mass_entry_point": "kvp_future_mass_chunked" if mass_ws is not None else "kvp_future_mass",
        "mass_pass_gpairs_per_s": round(pairs_layer / (mass_launch_ms * 1e-3) / 1e9, 3),
        "lse_pass_gpairs_per_s": round(lse_pairs / (lse_launch_ms * 1e-3) / 1e9, 3),
        "select_gbs": round(sel_bytes / (sel_launch_ms * 1e-3) / 1e9, 2),
        "roofline": {"kernel": "mass_kernel", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(wl.name)},
    }
    if not args.no_graph:
        out["graph"] = graph_replay(torch, step, args.steps, pairs_step,
                                    (lse_all, mass_all, keep_all))
    if not args.no_probe:
        probe = mfma_probe(torch)
        out["mfma_probe"] = probe
        out["roofline"]["measured_peak"] = probe["tflops"]
        out["roofline"]["frac_measured_peak"] = round(achieved / probe["tflops"], 4)
    if not args.no_extras:
        out["next_rows"] = next_rows(kvp, torch, wl, L, q_all, k_all, lse_all, stream)
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        gpu0 = (lse_all[0].cpu().numpy(), mass_all[0].cpu().numpy(),
                keep_all[:B].cpu().numpy())
        out["cpu_baseline"] = cpu_baseline(wl, li0, args.cpu_heads, gpu=gpu0)
        log(f"bench: parity of layer 0 on the oracle's sample: {out['cpu_baseline']['parity']}")
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
