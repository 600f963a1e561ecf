"""The entry points keep no state between calls (the no-allocation selection
aside), so two pipelines enqueued on two streams at once give the results
each gives alone, bit for bit: the causal LSE (LKV §3 Eq. 1, reused by KVpop
§3.2 Eq. 8), the future mass (KVpop §3.1 Eq. 2) through both calls, the
per-head mass and the keep-set (KVpop §3 Eq. 1, Eq. 4, Fig. 1) on the
register path and, for rows past 32768, on the split path, each stream with
its own workspaces.  Both streams have the default priority."""
import pytest
import torch

import future_attention_scoring_kvp_amd as kvp
import kvp_inputs
from parity import say, to_dev

pytestmark = pytest.mark.gpu


def pipeline(q, k, w, s, top, stream=None):
    mass_ws = None
    need = kvp.future_mass_workspace_bytes(q, k, w)
    if need:
        mass_ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    lse = kvp.lse_fwd(q, k, stream=stream)
    mass = kvp.future_mass(q, k, lse, w, stream=stream)
    mass_c = kvp.future_mass_chunked(q, k, lse, w, workspace=mass_ws, stream=stream)
    mass_h = kvp.future_mass_per_head(q, k, lse, w, stream=stream)
    keep = kvp.select_topk(mass, w, s, top, stream=stream)
    return [lse, mass, mass_c, mass_h, keep]


@pytest.mark.parametrize("S,top", [(4096, 512), (40000, 4000)])
def test_two_streams_at_once_equal_each_alone(S, top):
    layers = []
    for seed in (71, 72):
        wl = kvp_inputs.workload(2).with_(Hq=16, Hkv=4, S=S, seed=seed + S)
        li = kvp_inputs.make_layer(wl)
        layers.append((to_dev(li.q), to_dev(li.k), wl.window, wl.n_sink))
    say(f"[streams] S={S}: each pipeline alone")
    alone = []
    for q, k, w, s in layers:
        alone.append(pipeline(q, k, w, s, top))
        torch.cuda.synchronize()
    say(f"[streams] S={S}: both at once")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    both = []
    for (q, k, w, s), st in zip(layers, streams):
        with torch.cuda.stream(st):   # tensors allocated for this stream's work
            both.append(pipeline(q, k, w, s, top, stream=st))
    torch.cuda.synchronize()
    names = ["lse", "mass", "mass_chunked", "mass_per_head", "keep"]
    for a, b in zip(alone, both):
        for name, x, y in zip(names, a, b):
            assert torch.equal(x, y), f"S={S}: {name} differs when two streams run at once"
