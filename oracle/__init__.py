"""CPU oracle for the future-attention-mass path — TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper over ``kvp_oracle.cpp`` (plain fp64 C++).  Only the tests,
the smoke check and the benchmark's CPU-baseline leg import this package; the
GPU library and its Python binding never do.

Every function cites what it follows in the C++ source header:
  * logits / LSE: causal scaled softmax (LKV, §3 Preliminaries, Eq. 1) and the
    per-query log-normaliser reused by KVpop §3.2 (Eq. 8);
  * mass: KVpop §3.1 Eq. 2 un-normalised (App. B.1), summed over the group;
  * keep-set: KVpop §3 Eq. 1 budget, Eq. 4 eligible set, Fig. 1;
  * target scores: KVpop §3.1 Eq. 2-3, App. B.1-B.3; running cutoff: KVpop
    §3.2 (running top-k and its kernel);
  * block / future scores: ForesightKV §3.2 "Golden Eviction" with the
    appendix's block-level surrogate.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvp_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "libkvp_oracle.so")
_lock = threading.Lock()
_lib = None

DTYPE_BF16, DTYPE_F32_AS_BF16, DTYPE_F32_EXACT = 0, 1, 2


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH,
          extra_flags: Sequence[str] = ()) -> str:
    """Compile the oracle with g++ (-O3, no fast-math, no FMA contraction: plain IEEE fp64)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.check_call(["g++", "-O3", "-ffp-contract=off", "-std=c++17", "-fPIC", "-shared", "-pthread",
                               *extra_flags, src, "-o", tmp])
        os.replace(tmp, out)
    return out


def _bind(lib):
    i64, vp, dbl, cint = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double, ctypes.c_int
    lib.oracle_round_bf16.restype = cint
    lib.oracle_round_bf16.argtypes = [vp, i64, vp]
    lib.oracle_future_mass.restype = cint
    lib.oracle_future_mass.argtypes = [vp, vp, cint, i64, i64, i64, i64, i64, dbl, i64,
                                       i64, i64, i64, cint, vp, vp, vp, vp, vp]
    lib.oracle_lse_rows.restype = cint
    lib.oracle_lse_rows.argtypes = [vp, vp, cint, i64, i64, i64, i64, i64, dbl, vp, i64, cint, vp]
    lib.oracle_keep_count.restype = i64
    lib.oracle_keep_count.argtypes = [i64, i64, i64, i64]
    lib.oracle_select.restype = cint
    lib.oracle_select.argtypes = [vp, i64, i64, i64, i64, i64, i64, vp]
    if hasattr(lib, "oracle_sparse_lse"):
        lib.oracle_sparse_lse.restype = cint
        lib.oracle_sparse_lse.argtypes = [vp, vp, cint, i64, i64, i64, i64, i64, dbl, i64, vp, vp,
                                          cint, vp]
    if hasattr(lib, "oracle_block_scores"):
        lib.oracle_block_scores.restype = cint
        lib.oracle_block_scores.argtypes = [vp, vp, cint, i64, i64, i64, i64, i64, dbl, i64, i64,
                                            i64, cint, cint, vp, vp]
    if hasattr(lib, "oracle_running_cutoff"):
        lib.oracle_running_cutoff.restype = cint
        lib.oracle_running_cutoff.argtypes = [vp, i64, i64, i64, i64, i64, i64, vp, vp]
    return lib


def load(path: Optional[str] = None):
    """Load the oracle library (building it first if it is missing).  A
    non-default ``path`` loads a separately built variant (used by the tests
    that plant mistakes in a copy of the oracle)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _dtype_code(arr: np.ndarray, f32_exact: bool) -> int:
    if arr.dtype == np.uint16:
        return DTYPE_BF16
    if arr.dtype == np.float32:
        return DTYPE_F32_EXACT if f32_exact else DTYPE_F32_AS_BF16
    raise TypeError(f"unsupported input dtype {arr.dtype}")


def round_bf16(x: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    rc = lib.oracle_round_bf16(x.ctypes.data, x.size, out.ctypes.data)
    assert rc == 0
    return out


def future_mass(q: np.ndarray, k: np.ndarray, window: int, scale: float = 0.0, *,
                b_only: int = -1, h_only: int = -1, row_lo: int = 0,
                f32_exact: bool = False, nthreads: Optional[int] = None, lib=None,
                want_rowsum: bool = False, want_winmass: bool = False,
                want_per_head: bool = False) -> dict:
    """Dense causal softmax + future mass.  q: [B,Hq,S,D], k: [B,Hkv,S,D], as
    bf16 bit patterns (uint16) or float32 (rounded to bf16 unless
    ``f32_exact``).  Returns dict of fp64 arrays: lse [B,Hq,S], mass
    [B,Hkv,S] (+ rowsum, winmass, and the per-query-head masses mass_heads
    [B,Hq,S]).  Entries outside a b_only/h_only/row_lo restriction are NaN."""
    lib = lib or load()
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    if q.dtype != k.dtype:
        raise TypeError("q and k must have the same dtype")
    B, Hq, S, D = q.shape
    Bk, Hkv, Sk, Dk = k.shape
    if (B, S, D) != (Bk, Sk, Dk):
        raise ValueError("q/k shape mismatch")
    lse = np.full((B, Hq, S), np.nan)
    mass = np.full((B, Hkv, S), np.nan)
    rowsum = np.full((B, Hq, S), np.nan) if want_rowsum else None
    winmass = np.full((B, Hq, S), np.nan) if want_winmass else None
    mass_heads = np.full((B, Hq, S), np.nan) if want_per_head else None
    rc = lib.oracle_future_mass(
        q.ctypes.data, k.ctypes.data, _dtype_code(q, f32_exact), B, Hq, Hkv, S, D,
        float(scale), int(window), int(b_only), int(h_only), int(row_lo),
        nthreads or default_threads(), lse.ctypes.data, mass.ctypes.data,
        rowsum.ctypes.data if rowsum is not None else None,
        winmass.ctypes.data if winmass is not None else None,
        mass_heads.ctypes.data if mass_heads is not None else None)
    if rc != 0:
        raise ValueError(f"oracle_future_mass rejected the arguments (rc={rc})")
    out = {"lse": lse, "mass": mass}
    if rowsum is not None:
        out["rowsum"] = rowsum
    if winmass is not None:
        out["winmass"] = winmass
    if mass_heads is not None:
        out["mass_heads"] = mass_heads
    return out


def sparse_lse(q: np.ndarray, k: np.ndarray, window: int, rank: np.ndarray, cutoff: np.ndarray,
               scale: float = 0.0, *, f32_exact: bool = False, nthreads: Optional[int] = None,
               lib=None) -> np.ndarray:
    """KVpop §3.2 sparse log-normaliser [B, Hq, S] (fp64): the LSE of each
    query row over the running top-k pattern (window, sinks, eligible tokens
    of rank <= cutoff); rank / cutoff int32 [B, Hkv, S] from running_cutoff."""
    lib = lib or load()
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    rank = np.ascontiguousarray(rank, dtype=np.int32)
    cutoff = np.ascontiguousarray(cutoff, dtype=np.int32)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if rank.shape != (B, Hkv, S) or cutoff.shape != (B, Hkv, S):
        raise ValueError("rank and cutoff must be [B, Hkv, S]")
    out = np.empty((B, Hq, S), dtype=np.float64)
    rc = lib.oracle_sparse_lse(q.ctypes.data, k.ctypes.data, _dtype_code(q, f32_exact), B, Hq, Hkv,
                               S, D, float(scale), int(window), rank.ctypes.data,
                               cutoff.ctypes.data, nthreads or default_threads(), out.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_sparse_lse rejected the arguments (rc={rc})")
    return out


def block_count(S: int, block_start: int, block_len: int) -> int:
    """Number of query blocks [block_start + t L, block_start + (t+1) L) ∩ [0, S)."""
    return (S - block_start + block_len - 1) // block_len if S > block_start else 0


def block_scores(q: np.ndarray, k: np.ndarray, window: int, block_start: int, block_len: int,
                 scale: float = 0.0, *, per_head: bool = False, f32_exact: bool = False,
                 nthreads: Optional[int] = None, lib=None) -> dict:
    """ForesightKV Golden-Eviction scores in fp64 (§3.2 "Golden Eviction" and
    the appendix's block surrogate): ``block`` [B, U, n_blocks, S], the mean
    attention of every key over the rows of each query block and the query
    heads of each unit (KV head, or query head with ``per_head``), and
    ``future`` [B, U, n_blocks, S], its maximum over the blocks from t on."""
    lib = lib or load()
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    U = Hq if per_head else Hkv
    nb = block_count(S, block_start, block_len)
    block = np.full((B, U, nb, S), np.nan)
    future = np.full((B, U, nb, S), np.nan)
    rc = lib.oracle_block_scores(q.ctypes.data, k.ctypes.data, _dtype_code(q, f32_exact), B, Hq,
                                 Hkv, S, D, float(scale), int(window), int(block_start),
                                 int(block_len), 1 if per_head else 0,
                                 nthreads or default_threads(), block.ctypes.data,
                                 future.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_block_scores rejected the arguments (rc={rc})")
    return {"block": block, "future": future}


def lse_rows(q: np.ndarray, k: np.ndarray, rows: np.ndarray, scale: float = 0.0, *,
             f32_exact: bool = False, nthreads: Optional[int] = None, lib=None) -> np.ndarray:
    """LSE of selected (b, g, i) rows (int64 [n,3])."""
    lib = lib or load()
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    out = np.empty(rows.shape[0], dtype=np.float64)
    rc = lib.oracle_lse_rows(q.ctypes.data, k.ctypes.data, _dtype_code(q, f32_exact), B, Hq, Hkv,
                             S, D, float(scale), rows.ctypes.data, rows.shape[0],
                             nthreads or default_threads(), out.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_lse_rows rejected the arguments (rc={rc})")
    return out


def keep_count(S: int, window: int, n_sink: int, top_k: int, lib=None) -> int:
    lib = lib or load()
    return int(lib.oracle_keep_count(S, window, n_sink, top_k))


def select(mass: np.ndarray, window: int, n_sink: int, top_k: int, lib=None) -> np.ndarray:
    """Keep-set [B,Hkv,n_keep] (int32, ascending) from mass [B,Hkv,S]."""
    lib = lib or load()
    mass = np.ascontiguousarray(mass, dtype=np.float64)
    B, Hkv, S = mass.shape
    n_keep = keep_count(S, window, n_sink, top_k, lib)
    keep = np.empty((B, Hkv, max(n_keep, 0)), dtype=np.int32)
    rc = lib.oracle_select(mass.ctypes.data, B, Hkv, S, window, n_sink, top_k, keep.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_select failed (rc={rc})")
    return keep


def running_cutoff(score: np.ndarray, window: int, n_sink: int, top_k: int, lib=None):
    """KVpop §3.2 running top-k: (rank [B,Hkv,S], cutoff [B,Hkv,S]) int32.
    rank: position of each token t >= s in the order (priority descending,
    index ascending), -1 for sinks; cutoff[q]: rank of the k-th best eligible
    token at query q (Fenwick tree + binary lifting), S when fewer than k are
    eligible, -1 when k = 0."""
    lib = lib or load()
    score = np.ascontiguousarray(score, dtype=np.float64)
    B, H, S = score.shape
    rank = np.empty((B, H, S), dtype=np.int32)
    cutoff = np.empty((B, H, S), dtype=np.int32)
    rc = lib.oracle_running_cutoff(score.ctypes.data, B, H, S, window, n_sink, top_k,
                                   rank.ctypes.data, cutoff.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_running_cutoff failed (rc={rc})")
    return rank, cutoff


AGG_LOG_MEAN, AGG_MEAN_LOG, AGG_MAX_LOG = 0, 1, 2


def target_scores(mass: np.ndarray, window: int, n_kv_heads: int, *, per_head: bool = True,
                  group_size: Optional[int] = None, normalize: bool = True,
                  agg: int = AGG_MEAN_LOG, eps: float = 1e-6, query: int = -1,
                  decay_step: int = 1, log_gamma: Optional[np.ndarray] = None) -> np.ndarray:
    """KVpop target scores in fp64, [B, Hkv, S], following the page's steps:

    * count normalisation m / N_t with N_t = max(1, S - (t + w))  (§3.1 Eq. 2,
      App. B.2), or none (App. B.1);
    * log(eps + m) aggregated over the query heads g of each KV head
      (§3.1 Eq. 3): agg 0 = log of the group mean (App. B.1), 1 = mean of the
      logs, 2 = max of the logs;
    * with query >= 0 the temporal decay of App. B.3,
      r(q) = r + floor((q - t) / n) * log(gamma_h) for t <= q, and -inf for
      t > q (not generated yet).

    mass: [B, Hq, S] per-head masses (per_head) or [B, Hkv, S] group sums of
    group_size heads (only agg 0)."""
    with np.errstate(divide="ignore"):  # log(0) = -inf is the defined value for eps = 0
        return _target_scores(np.asarray(mass, dtype=np.float64), window, n_kv_heads, per_head,
                              group_size, normalize, agg, eps, query, decay_step, log_gamma)


def _target_scores(mass, window, n_kv_heads, per_head, group_size, normalize, agg, eps, query,
                   decay_step, log_gamma):
    B, H, S = mass.shape
    t = np.arange(S)
    n_t = np.maximum(1, S - (t + window)).astype(np.float64) if normalize else np.ones(S)
    if per_head:
        G = H // n_kv_heads
        m = mass.reshape(B, n_kv_heads, G, S) / n_t
        if agg == AGG_LOG_MEAN:
            r = np.log(eps + m.mean(axis=2))
        elif agg == AGG_MEAN_LOG:
            r = np.log(eps + m).mean(axis=2)
        elif agg == AGG_MAX_LOG:
            r = np.log(eps + m).max(axis=2)
        else:
            raise ValueError("unknown aggregation")
    else:
        if agg != AGG_LOG_MEAN:
            raise ValueError("group sums only support the log of the group mean")
        r = np.log(eps + mass / (group_size * n_t))
    if query >= 0:
        lg = np.asarray(log_gamma, dtype=np.float64).reshape(1, n_kv_heads, 1)
        steps = np.where(t <= query, (query - t) // decay_step, 0).astype(np.float64)
        r = r + steps * lg
        r = np.where(t <= query, r, -np.inf)
    return r


def static_priority(score: np.ndarray, decay_step: int, log_gamma: np.ndarray) -> np.ndarray:
    """Static token priorities of KVpop's running top-k (§3.2 "Running top-k
    sparse attention"; App. B.3 "Temporal Decay and Static Priorities"), fp64
    [B, Hkv, S].

    App. B.3 decays a token's score at query q by floor((q - t) / n) steps of
    log gamma_h.  Writing floor((q - t) / n) = floor(q / n) - floor(t / n) -
    [q mod n < t mod n], the part floor(q / n) log gamma_h is the same for
    every token at a given q, so the decayed order at q is the order of

        pi[t] = r[t] - floor(t / n) * log gamma_h,

    up to the last term, which is at most one decay step (|log gamma_h|) and
    vanishes for n = 1 and at every query with q mod n = n - 1.  The pages say
    only that the query-dependent part is shared up to the decay-step
    discretization; this is the reading taken.

    score: [B, Hkv, S] undecayed scores r (e.g. target_scores with query < 0);
    log_gamma: [Hkv] values of log gamma_h; decay_step: n >= 1."""
    r = np.asarray(score, dtype=np.float64)
    B, H, S = r.shape
    lg = np.asarray(log_gamma, dtype=np.float64).reshape(1, H, 1)
    steps = (np.arange(S) // int(decay_step)).astype(np.float64)
    return r - steps * lg


def _laplace_cdf(z):
    return np.where(z >= 0, 1.0 - 0.5 * np.exp(-np.abs(z)), 0.5 * np.exp(-np.abs(z)))


def soft_topk(x: np.ndarray, k, tau: float = 1.0):
    """LKV's Soft-TopK (§3.2 "The Differentiable Soft-TopK Operator", App. A.1)
    in fp64, row by row over the last axis: y_i = f(z_i - lam) with z = x / tau,
    f the Laplace CDF, and the threshold lam for which sum_i y_i = k.

    Following App. A.1: sort z descending; for a split m (the m largest
    elements in the saturation region) the budget equation is the quadratic
    S1 y^2 + 2 (k - m) y - S2 = 0 in y = e^lam, with S1 = sum_{i<=m} e^{-z_(i)}
    and S2 = sum_{i>m} e^{z_(i)}; the split is the one whose root lies between
    z_(m+1) and z_(m) (the first such m).  S1 and S2 are kept as logarithms
    (cumulative log-sum-exp), and their product, at most m (n - m), is formed
    from the sum of the logarithms.  The page keeps 1 <= m < n; m = 0 (lam
    above every element) and m = n (below every element) use the same
    equation's limits, y = S2 / (2k) and y = 2 (n - k) / S1.
    Returns (y, lam) with lam in units of z.  k: scalar or one per row, in
    (0, n)."""
    x = np.asarray(x, dtype=np.float64)
    rows = x.reshape(-1, x.shape[-1])
    n = rows.shape[1]
    kk = np.broadcast_to(np.asarray(k, dtype=np.float64), (rows.shape[0],))
    y = np.empty_like(rows)
    lam = np.empty(rows.shape[0])
    for r in range(rows.shape[0]):
        z = rows[r] / tau
        zs = np.sort(z)[::-1]
        m = np.arange(n + 1)
        # log S1(m) for m = 0..n (log 0 = -inf) and log S2(m)
        log_s1 = np.concatenate([[-np.inf], np.logaddexp.accumulate(-zs)])
        log_s2 = np.concatenate([np.logaddexp.accumulate(zs[::-1])[::-1], [-np.inf]])
        a = kk[r] - m
        with np.errstate(divide="ignore", invalid="ignore", over="ignore", under="ignore"):
            log_p = log_s1 + log_s2                          # log S1 S2; S1 S2 <= m (n - m)
            root = np.sqrt(a * a + np.exp(log_p))
            # log(y S1) with y S1 = sqrt(a^2 + S1 S2) - a, taken without
            # cancellation for a > 0 and without forming a vanishing product
            log_ys1 = np.where(a > 0, log_p - np.log(root + a),
                               np.where(a == 0, 0.5 * log_p, np.log(root - a)))
            cand = log_ys1 - log_s1
            cand[0] = log_s2[0] - math.log(2.0 * kk[r])       # m = 0
            cand[n] = math.log(2.0 * (n - kk[r])) - log_s1[n]  # m = n
        hi = np.concatenate([[np.inf], zs])                  # z_(m), m = 0..n
        lo = np.concatenate([zs, [-np.inf]])                 # z_(m+1)
        ok = np.isfinite(cand) & (lo <= cand) & (cand <= hi)
        if not ok.any():
            raise ValueError("no consistent split (k outside (0, n)?)")
        lam[r] = cand[np.argmax(ok)]
        y[r] = _laplace_cdf(z - lam[r])
    return y.reshape(x.shape), lam.reshape(x.shape[:-1])


def soft_topk_backward(x: np.ndarray, lam: np.ndarray, dy: np.ndarray, tau: float = 1.0):
    """Gradients of the Soft-TopK (LKV App. A.2, implicit function theorem):
    with f'(z) = e^{-|z|} / 2 and u_i = z_i - lam,
      d lam / d z_j = f'(u_j) / sum_i f'(u_i),   d lam / d k = -1 / sum_i f'(u_i),
    so for upstream dy:  dz_j = f'(u_j) (dy_j - sum_i dy_i f'(u_i) / sum_i f'(u_i)),
    dx = dz / tau and dk = sum_i dy_i f'(u_i) / sum_i f'(u_i)."""
    x = np.asarray(x, dtype=np.float64)
    lam = np.asarray(lam, dtype=np.float64)[..., None]
    dy = np.asarray(dy, dtype=np.float64)
    fp = 0.5 * np.exp(-np.abs(x / tau - lam))
    a = (dy * fp).sum(-1, keepdims=True)
    b = fp.sum(-1, keepdims=True)
    dz = fp * (dy - a / b)
    return dz / tau, (a / b)[..., 0]
