"""Future-attention mass for KV-cache eviction on AMD MI355X (gfx950).

Thin Python binding of ``libkvp.so`` (HIP kernels behind a C ABI declared in
``include/kvp.h``).  It only marshals arguments: it checks torch tensors'
device, dtype, shape and contiguity, and passes raw device pointers and the
current HIP stream to the library.  Every step of the computation runs in the
library's kernels; there is no fallback path.  If the library has not been
built, importing works but every call raises.

    lse  = lse_fwd(q, k)                          # [B, Hq, S]  fp32
    mass = future_mass(q, k, lse, window)         # [B, Hkv, S] fp32
    keep = select_topk(mass, window, n_sink, k)   # [B, Hkv, n_keep] int32

KVpop's training target from the masses:

    mh = future_mass_per_head(q, k, lse, window)  # [B, Hq, S] fp32
    r  = target_scores(mh, Hkv, window, agg=AGG_MEAN_LOG, eps=1e-6)   # [B, Hkv, S]

The running top-k mask of every query position:

    rank, cutoff = running_cutoff(r, window, n_sink, k)   # int32 [B, Hkv, S] each
    lse_s = lse_sparse(q, k, rank, cutoff, window)         # LSE of that sparse attention

ForesightKV's Golden-Eviction scores (query blocks of L rows after the first B):

    blk, fut = block_future_scores(q, k, lse, B, L)     # fp32 [B, Hkv, n_blocks, S] each

LKV's differentiable Soft-TopK over any score rows:

    y, lam = soft_topk(x, k, tau)                       # y sums to k per row
    dx, dk = soft_topk_backward(x, lam, dy, tau)
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

__all__ = ["lse_fwd", "lse_sparse", "future_mass", "future_mass_per_head", "future_mass_chunked",
           "future_mass_workspace_bytes", "target_scores",
           "static_priority", "select_topk", "select_topk_noalloc", "select_workspace_bytes", "keep_count",
           "running_cutoff", "block_count", "block_future_scores", "soft_topk",
           "soft_topk_backward", "KvpError", "library_path", "load_library", "AGG_LOG_MEAN",
           "AGG_MEAN_LOG", "AGG_MAX_LOG"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvp.so")
_lock = threading.Lock()
_lib = None

KVP_BF16, KVP_F32 = 0, 1
AGG_LOG_MEAN, AGG_MEAN_LOG, AGG_MAX_LOG = 0, 1, 2


class KvpError(RuntimeError):
    pass


class _Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32)]


def library_path() -> str:
    return LIB_PATH


def load_library():
    """Load libkvp.so (built by ``build.py`` / ``__graft_entry__.build()``)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise KvpError(f"libkvp.so is not built ({LIB_PATH}); run build() first")
            lib = ctypes.CDLL(LIB_PATH)
            vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
            lib.kvp_lse_fwd.restype = ctypes.c_int
            lib.kvp_lse_fwd.argtypes = [vp, vp, ctypes.c_int, _Dims, f32, vp, vp]
            lib.kvp_lse_sparse.restype = ctypes.c_int
            lib.kvp_lse_sparse.argtypes = [vp, vp, ctypes.c_int, _Dims, f32, vp, vp, i32, vp, vp]
            lib.kvp_future_mass.restype = ctypes.c_int
            lib.kvp_future_mass.argtypes = [vp, vp, vp, ctypes.c_int, _Dims, f32, i32, vp, vp]
            lib.kvp_future_mass_per_head.restype = ctypes.c_int
            lib.kvp_future_mass_workspace_bytes.restype = ctypes.c_size_t
            lib.kvp_future_mass_workspace_bytes.argtypes = [_Dims, ctypes.c_int, i32, i32]
            lib.kvp_future_mass_chunked.restype = ctypes.c_int
            lib.kvp_future_mass_chunked.argtypes = [vp, vp, vp, ctypes.c_int, _Dims, f32, i32, i32,
                                                    vp, vp, ctypes.c_size_t, vp]
            lib.kvp_future_mass_per_head.argtypes = [vp, vp, vp, ctypes.c_int, _Dims, f32, i32,
                                                     vp, vp]
            lib.kvp_target_scores.restype = ctypes.c_int
            lib.kvp_target_scores.argtypes = [vp, i32, _Dims, i32, i32, ctypes.c_int, f32, i32,
                                              i32, vp, vp, vp]
            lib.kvp_static_priority.restype = ctypes.c_int
            lib.kvp_static_priority.argtypes = [vp, _Dims, i32, vp, vp, vp]
            lib.kvp_keep_count.restype = i64
            lib.kvp_keep_count.argtypes = [i64, i64, i64, i64]
            lib.kvp_select_topk.restype = ctypes.c_int
            lib.kvp_select_topk.argtypes = [vp, _Dims, i32, i32, i32, vp, vp, ctypes.c_size_t,
                                            vp]
            lib.kvp_select_topk_noalloc.restype = ctypes.c_int
            lib.kvp_select_topk_noalloc.argtypes = [vp, _Dims, i32, i32, i32, vp, vp]
            lib.kvp_select_workspace_bytes.restype = ctypes.c_size_t
            lib.kvp_select_workspace_bytes.argtypes = [_Dims, i32]
            lib.kvp_block_count.restype = i64
            lib.kvp_block_count.argtypes = [i64, i64, i64]
            lib.kvp_block_future_scores.restype = ctypes.c_int
            lib.kvp_block_future_scores.argtypes = [vp, vp, vp, ctypes.c_int, _Dims, f32, i32, i32,
                                                    i32, i32, vp, vp, vp]
            lib.kvp_soft_topk_fwd.restype = ctypes.c_int
            lib.kvp_soft_topk_fwd.argtypes = [vp, i64, i32, vp, f32, vp, vp, vp]
            lib.kvp_soft_topk_bwd.restype = ctypes.c_int
            lib.kvp_soft_topk_bwd.argtypes = [vp, vp, vp, i64, i32, f32, vp, vp, vp]
            lib.kvp_running_cutoff_workspace_bytes.restype = ctypes.c_size_t
            lib.kvp_running_cutoff_workspace_bytes.argtypes = [_Dims, i32]
            lib.kvp_running_cutoff.restype = ctypes.c_int
            lib.kvp_running_cutoff.argtypes = [vp, _Dims, i32, i32, i32, vp, vp, vp,
                                               ctypes.c_size_t, vp]
            lib.kvp_status_string.restype = ctypes.c_char_p
            lib.kvp_status_string.argtypes = [ctypes.c_int]
            lib.kvp_abi_version.restype = i32
            lib.kvp_abi_version.argtypes = []
            _lib = lib
    return _lib


def _check(status: int, what: str):
    if status != 0:
        msg = load_library().kvp_status_string(status).decode()
        raise KvpError(f"{what}: {msg} (status {status})")


def _stream_ptr(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KVP_BF16
    if t.dtype == torch.float32:
        return KVP_F32
    raise KvpError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _require_device(*ts: torch.Tensor):
    for t in ts:
        if not t.is_cuda:
            raise KvpError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise KvpError("tensors must be contiguous")


def _dims(q: torch.Tensor, k: torch.Tensor) -> _Dims:
    if q.dim() != 4 or k.dim() != 4:
        raise KvpError("q and k must be [B, H, S, d]")
    B, Hq, S, D = q.shape
    Bk, Hkv, Sk, Dk = k.shape
    if (B, S, D) != (Bk, Sk, Dk):
        raise KvpError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)}")
    if q.dtype != k.dtype:
        raise KvpError("q and k must have the same dtype")
    return _Dims(B, Hq, Hkv, S, D)


def keep_count(seq_len: int, window: int, n_sink: int, top_k: int) -> int:
    return int(load_library().kvp_keep_count(seq_len, window, n_sink, top_k))


def lse_fwd(q: torch.Tensor, k: torch.Tensor, scale: float = 0.0,
            out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Per-query causal log-sum-exp, fp32 [B, Hq, S] (natural log)."""
    lib = load_library()
    _require_device(q, k)
    d = _dims(q, k)
    if out is None:
        out = torch.empty((d.batch, d.n_q_heads, d.seq_len), dtype=torch.float32, device=q.device)
    _require_device(out)
    if out.dtype != torch.float32 or tuple(out.shape) != (d.batch, d.n_q_heads, d.seq_len):
        raise KvpError("lse out must be fp32 [B, Hq, S]")
    _check(lib.kvp_lse_fwd(q.data_ptr(), k.data_ptr(), _dtype_code(q), d, float(scale),
                           out.data_ptr(), _stream_ptr(stream)), "kvp_lse_fwd")
    return out


def lse_sparse(q: torch.Tensor, k: torch.Tensor, rank: torch.Tensor, cutoff: torch.Tensor,
               window: int, scale: float = 0.0, out: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """Per-query LSE over the running top-k pattern (window, sinks and the
    eligible keys with rank <= cutoff), fp32 [B, Hq, S]; rank / cutoff int32
    [B, Hkv, S] from running_cutoff."""
    lib = load_library()
    _require_device(q, k, rank, cutoff)
    d = _dims(q, k)
    shape = (d.batch, d.n_kv_heads, d.seq_len)
    for t in (rank, cutoff):
        if t.dtype != torch.int32 or tuple(t.shape) != shape:
            raise KvpError("rank and cutoff must be int32 [B, Hkv, S]")
    if out is None:
        out = torch.empty((d.batch, d.n_q_heads, d.seq_len), dtype=torch.float32, device=q.device)
    _require_device(out)
    if out.dtype != torch.float32 or tuple(out.shape) != (d.batch, d.n_q_heads, d.seq_len):
        raise KvpError("lse out must be fp32 [B, Hq, S]")
    _check(lib.kvp_lse_sparse(q.data_ptr(), k.data_ptr(), _dtype_code(q), d, float(scale),
                              rank.data_ptr(), cutoff.data_ptr(), int(window), out.data_ptr(),
                              _stream_ptr(stream)), "kvp_lse_sparse")
    return out


def future_mass(q: torch.Tensor, k: torch.Tensor, lse: torch.Tensor, window: int,
                scale: float = 0.0, out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """Future-attention mass per key, summed over each GQA group, fp32 [B, Hkv, S]."""
    lib = load_library()
    _require_device(q, k, lse)
    d = _dims(q, k)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (d.batch, d.n_q_heads, d.seq_len):
        raise KvpError("lse must be fp32 [B, Hq, S]")
    if out is None:
        out = torch.empty((d.batch, d.n_kv_heads, d.seq_len), dtype=torch.float32, device=q.device)
    _require_device(out)
    if out.dtype != torch.float32 or tuple(out.shape) != (d.batch, d.n_kv_heads, d.seq_len):
        raise KvpError("mass out must be fp32 [B, Hkv, S]")
    _check(lib.kvp_future_mass(q.data_ptr(), k.data_ptr(), lse.data_ptr(), _dtype_code(q), d,
                               float(scale), int(window), out.data_ptr(), _stream_ptr(stream)),
           "kvp_future_mass")
    return out


def future_mass_workspace_bytes(q: torch.Tensor, k: torch.Tensor, window: int,
                                per_head: bool = False) -> int:
    """Bytes of workspace ``future_mass_chunked`` needs for these inputs (0: none)."""
    lib = load_library()
    return int(lib.kvp_future_mass_workspace_bytes(_dims(q, k), _dtype_code(q), int(window),
                                                   int(bool(per_head))))


def future_mass_chunked(q: torch.Tensor, k: torch.Tensor, lse: torch.Tensor, window: int,
                        per_head: bool = False, scale: float = 0.0,
                        workspace: Optional[torch.Tensor] = None,
                        out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The masses of ``future_mass`` (or ``future_mass_per_head``), short sequences
    spread over more workgroups through a workspace (allocated here when not given:
    a uint8 device tensor of ``future_mass_workspace_bytes`` bytes)."""
    lib = load_library()
    _require_device(q, k, lse)
    d = _dims(q, k)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (d.batch, d.n_q_heads, d.seq_len):
        raise KvpError("lse must be fp32 [B, Hq, S]")
    heads = d.n_q_heads if per_head else d.n_kv_heads
    if out is None:
        out = torch.empty((d.batch, heads, d.seq_len), dtype=torch.float32, device=q.device)
    _require_device(out)
    if out.dtype != torch.float32 or tuple(out.shape) != (d.batch, heads, d.seq_len):
        raise KvpError("mass out must be fp32 [B, Hkv or Hq, S]")
    need = int(lib.kvp_future_mass_workspace_bytes(d, _dtype_code(q), int(window),
                                                   int(bool(per_head))))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        _require_device(workspace)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(lib.kvp_future_mass_chunked(q.data_ptr(), k.data_ptr(), lse.data_ptr(), _dtype_code(q),
                                       d, float(scale), int(window), int(bool(per_head)),
                                       out.data_ptr(), ws_ptr or None, ws_bytes,
                                       _stream_ptr(stream)), "kvp_future_mass_chunked")
    return out


def future_mass_per_head(q: torch.Tensor, k: torch.Tensor, lse: torch.Tensor, window: int,
                         scale: float = 0.0, out: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """Future-attention mass per key for each query head, fp32 [B, Hq, S]."""
    lib = load_library()
    _require_device(q, k, lse)
    d = _dims(q, k)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (d.batch, d.n_q_heads, d.seq_len):
        raise KvpError("lse must be fp32 [B, Hq, S]")
    if out is None:
        out = torch.empty((d.batch, d.n_q_heads, d.seq_len), dtype=torch.float32, device=q.device)
    _require_device(out)
    if out.dtype != torch.float32 or tuple(out.shape) != (d.batch, d.n_q_heads, d.seq_len):
        raise KvpError("mass out must be fp32 [B, Hq, S]")
    _check(lib.kvp_future_mass_per_head(q.data_ptr(), k.data_ptr(), lse.data_ptr(),
                                        _dtype_code(q), d, float(scale), int(window),
                                        out.data_ptr(), _stream_ptr(stream)),
           "kvp_future_mass_per_head")
    return out


def target_scores(mass: torch.Tensor, n_kv_heads: int, window: int, *, per_head: bool = True,
                  group_size: Optional[int] = None,
                  normalize: bool = True, agg: int = AGG_MEAN_LOG, eps: float = 1e-6,
                  query: int = -1, decay_step: int = 1,
                  log_gamma: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """KVpop target scores fp32 [B, Hkv, S] from masses: [B, Hq, S] per head
    (``per_head``) or [B, Hkv, S] sums over groups of ``group_size`` query
    heads.  ``query >= 0`` applies the temporal decay with ``log_gamma``
    (fp32 [Hkv] on the GPU)."""
    lib = load_library()
    _require_device(mass)
    if mass.dtype != torch.float32 or mass.dim() != 3:
        raise KvpError("mass must be fp32 [B, H, S]")
    B, H, S = mass.shape
    Hkv = int(n_kv_heads)
    if Hkv < 1:
        raise KvpError("n_kv_heads must be >= 1")
    if per_head:
        if H % Hkv != 0:
            raise KvpError("query heads must be a multiple of n_kv_heads")
        Hq = H
    else:
        if H != Hkv or group_size is None or int(group_size) < 1:
            raise KvpError("group-sum masses must be [B, n_kv_heads, S] with group_size >= 1")
        Hq = Hkv * int(group_size)
    lg_ptr = None
    if query >= 0:
        if log_gamma is None:
            raise KvpError("decay needs log_gamma [Hkv]")
        _require_device(log_gamma)
        if log_gamma.dtype != torch.float32 or tuple(log_gamma.shape) != (Hkv,):
            raise KvpError("log_gamma must be fp32 [Hkv]")
        lg_ptr = log_gamma.data_ptr()
    if out is None:
        out = torch.empty((B, Hkv, S), dtype=torch.float32, device=mass.device)
    _require_device(out)
    if out.dtype != torch.float32 or tuple(out.shape) != (B, Hkv, S):
        raise KvpError("score out must be fp32 [B, Hkv, S]")
    d = _Dims(B, Hq, Hkv, S, 128)  # head_dim is not read
    _check(lib.kvp_target_scores(mass.data_ptr(), 1 if per_head else 0, d, int(window),
                                 1 if normalize else 0, int(agg), float(eps), int(query),
                                 int(decay_step), lg_ptr, out.data_ptr(), _stream_ptr(stream)),
           "kvp_target_scores")
    return out


def static_priority(score: torch.Tensor, decay_step: int, log_gamma: torch.Tensor,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Static priorities of the running top-k, fp32 [B, Hkv, S]:
    score - floor(t / decay_step) * log_gamma[h] (KVpop §3.2 with App. B.3).
    ``score`` fp32 [B, Hkv, S] undecayed; ``log_gamma`` fp32 [Hkv] on the GPU;
    ``out`` may be ``score`` itself."""
    lib = load_library()
    _require_device(score, log_gamma)
    if score.dtype != torch.float32 or score.dim() != 3:
        raise KvpError("score must be fp32 [B, Hkv, S]")
    B, H, S = score.shape
    if log_gamma.dtype != torch.float32 or tuple(log_gamma.shape) != (H,):
        raise KvpError("log_gamma must be fp32 [Hkv]")
    if out is None:
        out = torch.empty_like(score)
    _require_device(out)
    if out.dtype != torch.float32 or out.shape != score.shape:
        raise KvpError("priority out must be fp32 like score")
    _check(lib.kvp_static_priority(score.data_ptr(), _Dims(B, H, H, S, 128), int(decay_step),
                                   log_gamma.data_ptr(), out.data_ptr(), _stream_ptr(stream)),
           "kvp_static_priority")
    return out


def select_workspace_bytes(rows: int, seq_len: int, top_k: int = 0) -> int:
    """Bytes of device workspace select_topk needs for ``rows`` rows of
    ``seq_len`` scores (0 for rows of at most 32768)."""
    return int(load_library().kvp_select_workspace_bytes(_Dims(rows, 1, 1, seq_len, 128),
                                                         int(top_k)))


def select_topk(mass: torch.Tensor, window: int, n_sink: int, top_k: int,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """Keep-set per KV head, int32 [..., n_keep] ascending.  ``mass`` is
    [B, Hkv, S] (any leading dims are flattened into rows).  ``workspace`` (a
    uint8 GPU tensor of select_workspace_bytes bytes, 256-byte aligned) is
    allocated when needed and not given."""
    lib = load_library()
    _require_device(mass)
    if mass.dtype != torch.float32 or mass.dim() < 1:
        raise KvpError("mass must be fp32 [..., S]")
    S = mass.shape[-1]
    rows = mass.numel() // S if S else 0
    n_keep = keep_count(S, window, n_sink, top_k)
    if n_keep < 0:
        raise KvpError("window, n_sink and top_k must be >= 0")
    shape = (*mass.shape[:-1], n_keep)
    if out is None:
        out = torch.empty(shape, dtype=torch.int32, device=mass.device)
    _require_device(out)
    if out.dtype != torch.int32 or tuple(out.shape) != shape:
        raise KvpError(f"keep out must be int32 {shape}")
    d = _Dims(rows, 1, 1, S, 128)
    need = int(lib.kvp_select_workspace_bytes(d, int(top_k)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=mass.device)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _require_device(workspace)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(lib.kvp_select_topk(mass.data_ptr(), d, int(window), int(n_sink), int(top_k),
                               out.data_ptr(), ws_ptr, ws_bytes, _stream_ptr(stream)),
           "kvp_select_topk")
    return out


def select_topk_noalloc(mass: torch.Tensor, window: int, n_sink: int, top_k: int,
                        out: torch.Tensor, stream=None) -> torch.Tensor:
    """select_topk for callers that cannot allocate (e.g. under graph
    capture): ``out`` must be given; the split path's state lives in the
    library's own 32 MiB array per GPU, so calls that overlap on one GPU
    race."""
    lib = load_library()
    _require_device(mass, out)
    if mass.dtype != torch.float32 or mass.dim() < 1:
        raise KvpError("mass must be fp32 [..., S]")
    S = mass.shape[-1]
    rows = mass.numel() // S if S else 0
    shape = (*mass.shape[:-1], keep_count(S, window, n_sink, top_k))
    if out.dtype != torch.int32 or tuple(out.shape) != shape:
        raise KvpError(f"keep out must be int32 {shape}")
    _check(lib.kvp_select_topk_noalloc(mass.data_ptr(), _Dims(rows, 1, 1, S, 128), int(window),
                                       int(n_sink), int(top_k), out.data_ptr(),
                                       _stream_ptr(stream)), "kvp_select_topk_noalloc")
    return out


def running_cutoff(score: torch.Tensor, window: int, n_sink: int, top_k: int,
                   workspace: Optional[torch.Tensor] = None, stream=None):
    """Static ranks and per-query cutoff ranks of the running top-k, each
    int32 with the shape of ``score`` ([..., S], leading dims flattened into
    rows).  Token t >= n_sink is kept at query q iff t <= q - window and
    rank[t] <= cutoff[q].  ``workspace`` (a uint8 GPU tensor) is allocated
    when not given."""
    lib = load_library()
    _require_device(score)
    if score.dtype != torch.float32 or score.dim() < 1:
        raise KvpError("score must be fp32 [..., S]")
    if window < 0 or n_sink < 0 or top_k < 0:
        raise KvpError("window, n_sink and top_k must be >= 0")
    S = score.shape[-1]
    rows = score.numel() // S if S else 0
    d = _Dims(rows, 1, 1, S, 128)
    need = int(lib.kvp_running_cutoff_workspace_bytes(d, int(n_sink)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=score.device)
    _require_device(workspace)
    rank = torch.empty(score.shape, dtype=torch.int32, device=score.device)
    cutoff = torch.empty(score.shape, dtype=torch.int32, device=score.device)
    _check(lib.kvp_running_cutoff(score.data_ptr(), d, int(window), int(n_sink), int(top_k),
                                  rank.data_ptr(), cutoff.data_ptr(), workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(),
                                  _stream_ptr(stream)), "kvp_running_cutoff")
    return rank, cutoff


def block_count(seq_len: int, block_start: int, block_len: int) -> int:
    return int(load_library().kvp_block_count(seq_len, block_start, block_len))


def block_future_scores(q: torch.Tensor, k: torch.Tensor, lse: torch.Tensor, block_start: int,
                        block_len: int, window: int = 0, *, per_head: bool = False,
                        want_block: bool = True, scale: float = 0.0, stream=None):
    """Golden-Eviction block scores and future scores, fp32 [B, U, n_blocks, S]
    each (U = Hkv, or Hq with ``per_head``); ``block`` is None when
    ``want_block`` is false."""
    lib = load_library()
    _require_device(q, k, lse)
    d = _dims(q, k)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (d.batch, d.n_q_heads, d.seq_len):
        raise KvpError("lse must be fp32 [B, Hq, S]")
    nb = block_count(d.seq_len, block_start, block_len)
    if nb < 0:
        raise KvpError("block_start must be >= 0 and block_len >= 1")
    U = d.n_q_heads if per_head else d.n_kv_heads
    shape = (d.batch, U, nb, d.seq_len)
    fut = torch.empty(shape, dtype=torch.float32, device=q.device)
    blk = torch.empty(shape, dtype=torch.float32, device=q.device) if want_block else None
    _check(lib.kvp_block_future_scores(q.data_ptr(), k.data_ptr(), lse.data_ptr(),
                                       _dtype_code(q), d, float(scale), int(window),
                                       1 if per_head else 0, int(block_start), int(block_len),
                                       blk.data_ptr() if blk is not None else None,
                                       fut.data_ptr(), _stream_ptr(stream)),
           "kvp_block_future_scores")
    return blk, fut


def _rows_of(t: torch.Tensor):
    n = t.shape[-1]
    return (t.numel() // n if n else 0), n


def soft_topk(x: torch.Tensor, k, tau: float = 1.0, stream=None):
    """LKV Soft-TopK per row of ``x`` (fp32 [..., n]): returns (y, lam), y of
    the shape of x summing to k per row, lam fp32 [...] in units of x / tau.
    ``k`` is a float or an fp32 GPU tensor with one budget per row."""
    lib = load_library()
    _require_device(x)
    if x.dtype != torch.float32 or x.dim() < 1:
        raise KvpError("x must be fp32 [..., n]")
    rows, n = _rows_of(x)
    if not torch.is_tensor(k):
        k = torch.full(x.shape[:-1], float(k), dtype=torch.float32, device=x.device)
    _require_device(k)
    if k.dtype != torch.float32 or k.numel() != rows:
        raise KvpError("k must be fp32 with one budget per row")
    y = torch.empty_like(x)
    lam = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _check(lib.kvp_soft_topk_fwd(x.data_ptr(), rows, n, k.data_ptr(), float(tau), y.data_ptr(),
                                 lam.data_ptr(), _stream_ptr(stream)), "kvp_soft_topk_fwd")
    return y, lam


def soft_topk_backward(x: torch.Tensor, lam: torch.Tensor, dy: torch.Tensor, tau: float = 1.0,
                       stream=None):
    """Gradients of the Soft-TopK: (dx like x, dk fp32 [...])."""
    lib = load_library()
    _require_device(x, lam, dy)
    if x.dtype != torch.float32 or dy.dtype != torch.float32 or lam.dtype != torch.float32:
        raise KvpError("x, lam and dy must be fp32")
    rows, n = _rows_of(x)
    if dy.shape != x.shape or lam.numel() != rows:
        raise KvpError("dy must match x and lam must hold one value per row")
    dx = torch.empty_like(x)
    dk = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _check(lib.kvp_soft_topk_bwd(x.data_ptr(), lam.data_ptr(), dy.data_ptr(), rows, n, float(tau),
                                 dx.data_ptr(), dk.data_ptr(), _stream_ptr(stream)),
           "kvp_soft_topk_bwd")
    return dx, dk
