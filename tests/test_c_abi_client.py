"""libkvp.so from plain C (tests/c_abi_client.c): the boundary needs nothing
but include/kvp.h, device pointers from hipMalloc and a HIP stream.  On the
CPU the client checks the host functions and the argument checks that every
stage makes before launching anything; on the GPU it runs the path (causal
LSE, LKV §3 Eq. 1 as reused by KVpop §3.2 Eq. 8; future mass, KVpop §3.1
Eq. 2; keep-set, KVpop §3 Eq. 1 / Eq. 4 / Fig. 1) on inputs written by this
test, and its outputs must equal the Python binding's bit for bit and the
oracle's within the tolerances.  The binary is built by the build step
(tests/build_c_client.py), never by a test."""
import os
import subprocess

import numpy as np
import pytest

import kvp_inputs
import oracle
from parity import assert_keep, assert_lse, assert_mass, say

HERE = os.path.dirname(os.path.abspath(__file__))
CLIENT = os.path.join(HERE, "c_abi_client")


def client():
    if not os.path.exists(CLIENT):
        pytest.fail("tests/c_abi_client is not built (run the build step)")
    return CLIENT


def test_host_checks_from_c():
    if not os.path.exists(CLIENT):   # on the CPU a missing build is made here
        import __graft_entry__
        __graft_entry__.build()
    proc = subprocess.run([client(), "host"], capture_output=True, text=True, timeout=60)
    assert proc.returncode == 0, proc.stdout + proc.stderr
    assert "host checks ok" in proc.stdout


@pytest.mark.gpu
@pytest.mark.parametrize("B,Hq,Hkv,S,w,s,k", [
    (1, 8, 2, 3000, 100, 4, 300),      # short: the chunked call takes its workspace
    (1, 2, 1, 40000, 512, 4, 4000),    # rows past 32768: the split selection and its workspace
])
def test_path_from_c(tmp_path, B, Hq, Hkv, S, w, s, k):
    import torch

    import future_attention_scoring_kvp_amd as kvp
    from parity import to_dev

    D = 128
    wl = kvp_inputs.workload(2).with_(B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, window=w, n_sink=s,
                                      top_k=k, seed=3131 + S)
    li = kvp_inputs.make_layer(wl)
    qf, kf = tmp_path / "q.bin", tmp_path / "k.bin"
    li.q.tofile(qf)
    li.k.tofile(kf)
    say(f"[c client] B={B} Hq={Hq} Hkv={Hkv} S={S} w={w} s={s} k={k}")
    proc = subprocess.run([client(), "run", *map(str, (B, Hq, Hkv, S, D, w, s, k)), str(qf),
                           str(kf), str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert proc.returncode == 0, proc.stdout + proc.stderr
    n_keep = kvp.keep_count(S, w, s, k)
    lse_c = np.fromfile(tmp_path / "lse.bin", np.float32).reshape(B, Hq, S)
    mass_c = np.fromfile(tmp_path / "mass.bin", np.float32).reshape(B, Hkv, S)
    mass_cc = np.fromfile(tmp_path / "mass_chunked.bin", np.float32).reshape(B, Hkv, S)
    keep_c = np.fromfile(tmp_path / "keep.bin", np.int32).reshape(B, Hkv, n_keep)

    # the same calls through the Python binding: the same bits
    q, kk = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, kk)
    mass = kvp.future_mass(q, kk, lse, w)
    mass2 = kvp.future_mass_chunked(q, kk, lse, w)
    keep = kvp.select_topk(mass, w, s, k)
    torch.cuda.synchronize()
    assert np.array_equal(lse_c, lse.cpu().numpy())
    assert np.array_equal(mass_c, mass.cpu().numpy())
    assert np.array_equal(mass_cc, mass2.cpu().numpy())
    assert np.array_equal(keep_c, keep.cpu().numpy())

    # and the oracle (the last KV head in full)
    h = Hkv - 1
    ref = oracle.future_mass(li.q, li.k, w, b_only=0, h_only=h)
    G = Hq // Hkv
    assert_lse(lse_c[:, h * G:(h + 1) * G], ref["lse"][:, h * G:(h + 1) * G], "C client lse")
    assert_mass(mass_c[:, h], ref["mass"][:, h], "C client mass")
    assert_mass(mass_cc[:, h], ref["mass"][:, h], "C client chunked mass")
    exact = oracle.select(ref["mass"][:, h:h + 1], w, s, k)
    assert_keep(keep_c[:, h:h + 1], ref["mass"][:, h:h + 1], w, s, k, exact, "C client keep")
