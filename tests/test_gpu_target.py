"""GPU parity of KVpop's target scores: per-query-head masses, the target
epilogue (count normalisation, log(eps + m), aggregation over the group,
temporal decay) and selection on signed scores, against the CPU oracle."""
import math

import numpy as np
import pytest
import torch

import future_attention_scoring_kvp_amd as kvp
import kvp_inputs
import oracle
from parity import MASS_ATOL, MASS_RTOL, assert_keep, assert_mass, say, to_dev

pytestmark = pytest.mark.gpu

# Scores computed by the GPU from its own masses: a relative mass error e
# moves log(eps + m) by at most about e, so the mass tolerance becomes an
# absolute one on the scores.
SCORE_ATOL = 2.5e-3


def score_tol(v):
    return SCORE_ATOL


def close_scores(got, ref, atol, rtol, what):
    got = got.astype(np.float64)
    both_inf = np.isneginf(got) & np.isneginf(ref)
    with np.errstate(invalid="ignore"):  # -inf - -inf where both_inf already decides
        bad = ~both_inf & ~(np.abs(got - ref) <= atol + rtol * np.abs(ref))
    assert not bad.any(), (f"{what}: {int(bad.sum())} mismatches, e.g. "
                           f"{got[bad][:3]} vs {ref[bad][:3]}")


@pytest.mark.parametrize("B,Hq,Hkv,S,D,w", [(1, 4, 1, 300, 128, 20), (2, 8, 2, 1000, 128, 64),
                                            (1, 4, 4, 257, 64, 0), (1, 8, 1, 4097, 128, 128)])
def test_per_head_mass(B, Hq, Hkv, S, D, w):
    wl = kvp_inputs.workload(2).with_(B=B, Hq=Hq, Hkv=Hkv, S=S, D=D, seed=100 + S)
    li = kvp_inputs.make_layer(wl)
    say(f"[target] per-head mass B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} w={w}")
    q, k = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, k)
    mh = kvp.future_mass_per_head(q, k, lse, w)
    mg = kvp.future_mass(q, k, lse, w)
    torch.cuda.synchronize()
    ref = oracle.future_mass(li.q, li.k, w, want_per_head=True)
    assert_mass(mh.cpu().numpy(), ref["mass_heads"], "per-head mass")
    # the group mass is the sum of its heads' masses (same kernels, fp32 sums)
    G = Hq // Hkv
    np.testing.assert_allclose(mh.view(B, Hkv, G, S).double().sum(2).cpu().numpy(),
                               mg.double().cpu().numpy(), rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("per_head,agg,normalize,eps,query", [
    (1, oracle.AGG_MEAN_LOG, 1, 1e-6, -1), (1, oracle.AGG_MAX_LOG, 1, 1e-6, -1),
    (1, oracle.AGG_LOG_MEAN, 0, 1e-4, -1), (0, oracle.AGG_LOG_MEAN, 1, 1e-6, -1),
    (1, oracle.AGG_MEAN_LOG, 1, 0.0, -1), (1, oracle.AGG_MEAN_LOG, 1, 1e-6, 700),
    (0, oracle.AGG_LOG_MEAN, 0, 1e-6, 999)])
def test_target_epilogue_on_the_same_masses(per_head, agg, normalize, eps, query):
    """The epilogue alone, on masses both sides read identically (fp32)."""
    rng = np.random.default_rng(5 + agg + 2 * per_head)
    B, Hkv, G, S, w, n = 2, 3, 4, 1000, 50, 16
    H = Hkv * G if per_head else Hkv
    mass = (rng.random((B, H, S)) ** 4 * 3).astype(np.float32)
    mass[..., S - w:] = 0.0
    lg = np.log(np.array([0.5, 0.8, 0.95])).astype(np.float32)
    say(f"[target] epilogue per_head={per_head} agg={agg} normalize={normalize} eps={eps} q={query}")
    got = kvp.target_scores(torch.from_numpy(mass).cuda(), Hkv, w, per_head=bool(per_head),
                            group_size=G, normalize=bool(normalize), agg=agg, eps=eps,
                            query=query, decay_step=n,
                            log_gamma=torch.from_numpy(lg).cuda()).cpu().numpy()
    ref = oracle.target_scores(mass.astype(np.float64), w, Hkv, per_head=bool(per_head),
                               group_size=G, normalize=bool(normalize), agg=agg, eps=eps,
                               query=query, decay_step=n, log_gamma=lg.astype(np.float64))
    close_scores(got, ref, 1e-5, 1e-5, "epilogue")


@pytest.mark.parametrize("wl_no,agg", [(2, oracle.AGG_MEAN_LOG), (2, oracle.AGG_LOG_MEAN)])
def test_target_end_to_end_keep_set(wl_no, agg):
    """GPU masses -> GPU targets -> GPU keep-set, against the oracle chain."""
    wl = kvp_inputs.workload(wl_no).with_(S=2048, seed=31)
    li = kvp_inputs.make_layer(wl)
    w, s, k = wl.window, wl.n_sink, wl.top_k
    say(f"[target] end to end S={wl.S} agg={agg}")
    q, kk = to_dev(li.q), to_dev(li.k)
    lse = kvp.lse_fwd(q, kk)
    mh = kvp.future_mass_per_head(q, kk, lse, w)
    r = kvp.target_scores(mh, wl.Hkv, w, agg=agg, eps=1e-6)
    keep = kvp.select_topk(r, w, s, k)
    torch.cuda.synchronize()
    ref_heads = oracle.future_mass(li.q, li.k, w, want_per_head=True)["mass_heads"]
    ref_r = oracle.target_scores(ref_heads, w, wl.Hkv, agg=agg, eps=1e-6)
    got_r = r.cpu().numpy()
    # the window has zero mass: log(eps) exactly on both sides
    close_scores(got_r, ref_r, SCORE_ATOL, 0.0, "targets")
    exact = oracle.select(ref_r, w, s, k)
    assert_keep(keep.cpu().numpy(), ref_r, w, s, k, exact, "target keep-set", score_tol)
    # exact on the GPU's own scores
    assert np.array_equal(keep.cpu().numpy(), oracle.select(got_r.astype(np.float64), w, s, k))


def test_select_signed_scores_exact():
    """Selection on scores of either sign, with exact ties, -0 / +0 and -inf,
    is bit-identical to the oracle's full sort."""
    rng = np.random.default_rng(9)
    for S, w, s, k in [(3000, 100, 4, 500), (777, 0, 0, 400), (4096, 128, 4, 512)]:
        say(f"[target] signed select S={S}")
        m = (np.round(rng.standard_normal((2, 3, S)) * 8) / 8).astype(np.float32)
        m[0, 0, ::7] = -np.inf
        m[0, 1, ::5] = -0.0
        m[0, 1, 1::5] = 0.0
        m[1, 0] = -np.abs(m[1, 0]) - 1.0   # all negative
        keep = kvp.select_topk(torch.from_numpy(m).cuda(), w, s, k).cpu().numpy()
        ref = oracle.select(m.astype(np.float64), w, s, k)
        assert np.array_equal(keep, ref)
