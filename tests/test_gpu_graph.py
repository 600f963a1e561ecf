"""The path captured into a HIP graph (torch.cuda.graph) and replayed: the
entry points only enqueue kernels on the caller's stream (no allocation, no
memset, no host synchronisation), with caller-owned outputs and workspaces,
so a capture records the same launches.  Each graph is replayed several
times, with other eager library work and synchronisations between the
replays, and every replay must give the eager result bit for bit: the causal
LSE (LKV §3 Eq. 1, reused by KVpop §3.2 Eq. 8), the future mass (KVpop §3.1
Eq. 2) through the chunked call with its workspace, the keep-set (KVpop §3
Eq. 1 and Eq. 4, Fig. 1) on the register path and on the split path with its
workspace, and the chain of the next rows: per-head masses, the target and
static priorities (App. B.1-B.3), the running cutoff, the sparse LSE and the
Golden-Eviction block scores."""
import pytest
import torch

import future_attention_scoring_kvp_amd as kvp
import kvp_inputs
from parity import say, to_dev

pytestmark = pytest.mark.gpu


def replays_match(g, outs, refs, dirty, n=3):
    for r in range(n):
        dirty(r)                      # other eager work on the same stream
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, o, e in zip(refs.keys(), outs, refs.values()):
            assert torch.equal(o, e), f"replay {r}: {name} differs from the eager result"


def test_short_path_chunked_mass_and_register_select():
    wl = kvp_inputs.workload(2)
    li = kvp_inputs.make_layer(wl)
    q, k = to_dev(li.q), to_dev(li.k)
    w, s, top = wl.window, wl.n_sink, wl.top_k
    li2 = kvp_inputs.make_layer(wl.with_(seed=99))
    q2, k2 = to_dev(li2.q), to_dev(li2.k)
    need = kvp.future_mass_workspace_bytes(q, k, w)
    assert need > 0
    say(f"[graph] 4K layer, chunked mass workspace {need} bytes")
    # eager reference (also loads every kernel before the capture)
    lse_e = kvp.lse_fwd(q, k)
    mass_e = kvp.future_mass_chunked(q, k, lse_e, w)
    keep_e = kvp.select_topk(mass_e, w, s, top)
    torch.cuda.synchronize()
    # static buffers for the graph
    lse_g = torch.empty_like(lse_e)
    mass_g = torch.empty_like(mass_e)
    keep_g = torch.empty_like(keep_e)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kvp.lse_fwd(q, k, out=lse_g)
        kvp.future_mass_chunked(q, k, lse_g, w, workspace=ws, out=mass_g)
        kvp.select_topk(mass_g, w, s, top, out=keep_g)

    def dirty(r):
        l2 = kvp.lse_fwd(q2, k2)
        kvp.future_mass_chunked(q2, k2, l2, w // (r + 1))
        lse_g.fill_(float("nan"))
        mass_g.fill_(-1.0)
        keep_g.fill_(-7)

    replays_match(g, (lse_g, mass_g, keep_g), {"lse": lse_e, "mass": mass_e, "keep": keep_e}, dirty)


def test_next_rows_chain_and_split_select():
    """Rows of 40000 keys (the split selection path, with its workspace), the
    per-head mass, target, static priorities, running cutoff, sparse LSE and
    block scores, all in one graph."""
    wl = kvp_inputs.workload(4).with_(Hq=8, Hkv=2, S=40000, window=512, top_k=4000, seed=4040)
    li = kvp_inputs.make_layer(wl)
    q, k = to_dev(li.q), to_dev(li.k)
    w, s, top, Hkv = wl.window, wl.n_sink, wl.top_k, wl.Hkv
    log_gamma = torch.log(torch.linspace(0.9, 0.99, Hkv, device="cuda", dtype=torch.float32))
    assert kvp.select_workspace_bytes(wl.B * Hkv, wl.S, top) > 0
    # workspaces big enough for the graph's calls and the eager ones between replays
    sel_need = max(kvp.select_workspace_bytes(wl.B * Hkv, wl.S, top),
                   kvp.select_workspace_bytes(3, 50000, 7000))
    lib = kvp.load_library()
    cut_need = max(int(lib.kvp_running_cutoff_workspace_bytes(kvp._Dims(wl.B * Hkv, 1, 1, wl.S, 128), s)),
                   int(lib.kvp_running_cutoff_workspace_bytes(kvp._Dims(3, 1, 1, 50000, 128), 4)), 1)
    say(f"[graph] S={wl.S}: split select workspace {sel_need} bytes")

    def chain(sel_ws, cut_ws):
        lse = kvp.lse_fwd(q, k)
        mass = kvp.future_mass(q, k, lse, w)
        keep = kvp.select_topk(mass, w, s, top, workspace=sel_ws)
        mh = kvp.future_mass_per_head(q, k, lse, w)
        tgt = kvp.target_scores(mh, Hkv, w)
        pri = kvp.static_priority(tgt, 64, log_gamma)
        rank, cut = kvp.running_cutoff(pri, w, s, top, workspace=cut_ws)
        lsp = kvp.lse_sparse(q, k, rank, cut, w)
        blk, fut = kvp.block_future_scores(q, k, lse, 1024, 256, w)
        return {"lse": lse, "mass": mass, "keep": keep, "mass_heads": mh, "target": tgt,
                "priority": pri, "rank": rank, "cutoff": cut, "lse_sparse": lsp,
                "block": blk, "future": fut}

    sel_ws = torch.empty(sel_need, dtype=torch.uint8, device="cuda")
    cut_ws = torch.empty(cut_need, dtype=torch.uint8, device="cuda")
    refs = chain(sel_ws, cut_ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = chain(sel_ws, cut_ws)

    def dirty(r):
        # eager calls that reuse both workspaces with other shapes and data
        m = torch.rand(3, 50000, device="cuda")
        kvp.select_topk(m, 100 * (r + 1), 4, 7000, workspace=sel_ws)
        kvp.running_cutoff(m, 64, 4, 1000 + r, workspace=cut_ws)
        for o in outs.values():
            o.fill_(3 if o.dtype == torch.int32 else float("nan"))

    replays_match(g, tuple(outs.values()), refs, dirty)
