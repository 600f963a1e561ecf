"""Write oracle_snapshot_s96.json: the CPU oracle's output on one small seeded
input (the tiny workload's recipe at S=96, w=8, s=4, k=12).  Calls only the
oracle and the input generator; rerun it only when the oracle's arithmetic is
deliberately changed (and name the passage that justifies the change)."""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import kvp_inputs  # noqa: E402
import oracle  # noqa: E402

WL = dict(S=96, window=8, n_sink=4, top_k=12)


def compute():
    wl = kvp_inputs.workload(1).with_(S=WL["S"], window=WL["window"], n_sink=WL["n_sink"],
                                      top_k=WL["top_k"])
    li = kvp_inputs.make_layer(wl)
    out = oracle.future_mass(li.q, li.k, wl.window)
    keep = oracle.select(out["mass"], wl.window, wl.n_sink, wl.top_k)
    return {
        "workload": "tiny recipe (fp32 N(0,1), rounded to bf16), S=96, d=64, seed 20262202",
        **WL,
        "lse": out["lse"][0, 0].tolist(),
        "mass": out["mass"][0, 0].tolist(),
        "keep": keep[0, 0].tolist(),
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "oracle_snapshot_s96.json"), "w") as f:
        json.dump(compute(), f, indent=1)
