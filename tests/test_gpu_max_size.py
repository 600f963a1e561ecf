"""The largest supported sequence, S = 2^22 (one query / KV head, d = 128):
the byte offsets of a head reach 2^30 (bf16) and the kernels' 32-bit index
arithmetic is at its widest.  The oracle's mass pass does not run at this
size; the results are checked on sampled rows and keys recomputed in fp64
from the definition (the last 64 rows and the 64 keys that only they reach
entirely independently of the GPU's LSE), by properties that hold at any size,
and the keep-set bit for bit against the oracle's full sort of the GPU's
masses."""
import math

import numpy as np
import pytest
import torch

import future_attention_scoring_kvp_amd as kvp
import oracle
from parity import LSE_ATOL, MASS_ATOL, MASS_RTOL, say

pytestmark = pytest.mark.gpu

S = 1 << 22
D = 128


def bf16_randn(gen, shape):
    return torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def test_max_sequence_length():
    gen = torch.Generator(device="cuda").manual_seed(20261202)
    q = bf16_randn(gen, (1, 1, S, D))
    k = bf16_randn(gen, (1, 1, S, D))
    say(f"[max size] S={S}")
    lse = kvp.lse_fwd(q, k)
    mass0 = kvp.future_mass(q, k, lse, 0)          # H2O: every row's mass, total S
    w, s, top = 4096, 4, 1 << 20
    mass = kvp.future_mass(q, k, lse, w)
    keep = kvp.select_topk(mass, w, s, top)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(lse)) and torch.all(torch.isfinite(mass))

    # with w = 0 every softmax row adds 1 in all: total = S up to fp32 rounding
    total = mass0.double().sum().item()
    assert abs(total - S) <= 1e-4 * S, total
    assert torch.all(mass[0, 0, S - w:] == 0)

    qf = q[0, 0].float().cpu().numpy().astype(np.float64)
    kf = k[0, 0].float().cpu().numpy().astype(np.float64)
    lse_np = lse[0, 0].cpu().numpy().astype(np.float64)
    scale = 1.0 / math.sqrt(D)
    # sampled rows: the causal LSE from its definition
    for i in (0, 1, 65535, 1 << 21, S - 1):
        logits = kf[: i + 1] @ qf[i] * scale
        m = logits.max()
        ref = m + math.log(np.exp(logits - m).sum())
        assert abs(lse_np[i] - ref) <= LSE_ATOL, (i, lse_np[i], ref)
    # sampled keys: the future mass from its definition, with the GPU's LSE
    m_np = mass[0, 0].cpu().numpy().astype(np.float64)
    for j in (0, 12345, S - w - 1):
        rows = np.arange(j + w, S)
        p = np.exp(qf[rows] @ kf[j] * scale - lse_np[rows])
        ref = p.sum()
        assert abs(m_np[j] - ref) <= MASS_ATOL + MASS_RTOL * ref, (j, m_np[j], ref)

    # keys just below the window, S-w-64 <= j < S-w, have only the last 64 rows
    # as future queries: their masses and those rows' LSE from the definition,
    # independent of the GPU's LSE
    tail = np.arange(S - 64, S)
    logits = (kf @ qf[tail].T) * scale                      # [S, 64]
    causal = np.arange(S)[:, None] <= tail[None, :]
    logits = np.where(causal, logits, -np.inf)
    mx = logits.max(axis=0)
    lse_ref = mx + np.log(np.exp(logits - mx).sum(axis=0))
    err = np.abs(lse_np[tail] - lse_ref).max()
    assert err <= LSE_ATOL, err
    keys = np.arange(S - w - 64, S - w)
    p = np.exp(logits[keys] - lse_ref)                       # [64 keys, 64 rows]
    p = np.where(tail[None, :] >= keys[:, None] + w, p, 0.0)
    ref_tail = p.sum(axis=1)
    np.testing.assert_array_less(np.abs(m_np[keys] - ref_tail),
                                 MASS_ATOL + MASS_RTOL * ref_tail + 1e-30)
    del logits, causal, p

    # keep-set: bit-exact against the oracle's full sort of the GPU's masses
    n_keep = kvp.keep_count(S, w, s, top)
    kp = keep[0, 0].cpu().numpy()
    assert kp.shape == (n_keep,)
    assert np.array_equal(kp, oracle.select(m_np.reshape(1, 1, S), w, s, top)[0, 0])
