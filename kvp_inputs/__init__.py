"""Seeded synthetic Q/K inputs for the future-attention-mass path.

Shared by the CPU oracle's tests and by the GPU path; it holds none of the
method's arithmetic, only input generation.  Values are standard normals from
a counter-based SplitMix64 + Box-Muller stream (``gen.c``), shaped by the
workload recipes below and rounded to bfloat16 (round to nearest even) for the
bf16 workloads.

Workloads (one layer of one model family each, Q and K after RoPE):

=====  ====================  ==========================================================
no.    name                  recipe
=====  ====================  ==========================================================
1      tiny                  B=1, Hq=Hkv=1, S=256, d=64, fp32 N(0,1); w=16, s=4, k=32
2      gqa4k                 B=1, 32/8 heads, S=4096, d=128, bf16 N(0,1); K row 0 x4,
                             1% of keys (positions drawn from [1,S)) x3; w=128, s=4, k=512
3      llama8b_16k           B=4, 32/8 heads, S=16384, d=128, bf16 N(0,1) + 0.5*U_h a_{b,t}
                             (per-KV-head rank-4 U_h, per-token a_{b,t}, both N(0,1));
                             w=256, s=4, k=1024
4      qwen3_4b_32k_stack    36 layers, B=1, 32/8 heads, S=32768, d=128, bf16 N(0,1) seeded
                             per layer; 1% heavy keys x3; w=512, s=4, k=16384
5      llama70b_128k         B=1, 64/8 heads, S=131072, d=128, bf16 N(0,1); K row 0 x4,
                             0.5% heavy keys x3; w=1024, s=4, k=2048
=====  ====================  ==========================================================

The seed of layer ``l`` of workload ``n`` is ``20261202 + 1000*n + l``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkvp_inputs.so")
_SRC = os.path.join(_HERE, "gen.c")
_lock = threading.Lock()
_lib = None

TAG_Q, TAG_K, TAG_U, TAG_A, TAG_HEAVY = 1, 2, 3, 4, 5
BASE_SEED = 20261202


def build(force: bool = True) -> str:
    """Compile gen.c into libkvp_inputs.so next to it (gcc, -O2)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            u64, i64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
            lib.kvpgen_stream_key.restype = u64
            lib.kvpgen_stream_key.argtypes = [u64, u64]
            lib.kvpgen_u64.restype = u64
            lib.kvpgen_u64.argtypes = [u64, u64]
            lib.kvpgen_normal.restype = ctypes.c_double
            lib.kvpgen_normal.argtypes = [u64, u64]
            lib.kvpgen_normals_f64.restype = None
            lib.kvpgen_normals_f64.argtypes = [u64, u64, i64, vp]
            lib.kvpgen_choose.restype = ctypes.c_int
            lib.kvpgen_choose.argtypes = [u64, i64, i64, i64, vp]
            lib.kvpgen_tensor.restype = ctypes.c_int
            lib.kvpgen_tensor.argtypes = [u64, i64, i64, i64, i64, vp, vp, vp, ctypes.c_int,
                                          ctypes.c_double, i64, ctypes.c_int, vp, ctypes.c_int]
            _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def stream_key(seed: int, tag: int) -> int:
    return int(_load().kvpgen_stream_key(seed & (2**64 - 1), tag))


def normals(key: int, count: int, offset: int = 0) -> np.ndarray:
    out = np.empty(count, dtype=np.float64)
    if count:
        _load().kvpgen_normals_f64(key, offset, count, out.ctypes.data)
    return out


def choose(key: int, lo: int, hi: int, count: int) -> np.ndarray:
    out = np.empty(max(count, 1), dtype=np.int64)
    rc = _load().kvpgen_choose(key, lo, hi, count, out.ctypes.data)
    if rc != 0:
        raise ValueError(f"choose({lo},{hi},{count}) failed: {rc}")
    return out[:count]


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class Workload:
    number: int
    name: str
    B: int
    Hq: int
    Hkv: int
    S: int
    D: int
    window: int
    n_sink: int
    top_k: int
    layers: int = 1
    dtype: str = "bf16"              # "bf16" or "f32"
    sink_scale: float = 1.0          # scale of K row 0
    heavy_frac: float = 0.0          # fraction of positions in [1, S) whose K rows are scaled
    heavy_scale: float = 1.0
    lowrank_rank: int = 0            # per-KV-head shared component U_h a_{b,t}
    lowrank_scale: float = 0.0
    seed: Optional[int] = None       # overrides BASE_SEED + 1000*number (+ layer)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def layer_seed(self, layer: int) -> int:
        base = self.seed if self.seed is not None else BASE_SEED + 1000 * self.number
        return base + layer

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "tiny", 1, 1, 1, 256, 64, 16, 4, 32, dtype="f32"),
    2: Workload(2, "gqa4k", 1, 32, 8, 4096, 128, 128, 4, 512,
                sink_scale=4.0, heavy_frac=0.01, heavy_scale=3.0),
    3: Workload(3, "llama8b_16k", 4, 32, 8, 16384, 128, 256, 4, 1024,
                lowrank_rank=4, lowrank_scale=0.5),
    4: Workload(4, "qwen3_4b_32k_stack", 1, 32, 8, 32768, 128, 512, 4, 16384, layers=36,
                heavy_frac=0.01, heavy_scale=3.0),
    5: Workload(5, "llama70b_128k", 1, 64, 8, 131072, 128, 1024, 4, 2048,
                sink_scale=4.0, heavy_frac=0.005, heavy_scale=3.0),
}


def workload(n: int) -> Workload:
    return WORKLOADS[n]


@dataclass
class LayerInputs:
    wl: Workload
    layer: int
    q: np.ndarray                     # [B,Hq,S,D] uint16 (bf16 bits) or float32
    k: np.ndarray                     # [B,Hkv,S,D]
    heavy: np.ndarray = field(default_factory=lambda: np.empty(0, np.int64))

    @property
    def dtype(self) -> str:
        return self.wl.dtype

    def q_f32(self) -> np.ndarray:
        return self.q if self.wl.dtype == "f32" else bf16_bits_to_f32(self.q)

    def k_f32(self) -> np.ndarray:
        return self.k if self.wl.dtype == "f32" else bf16_bits_to_f32(self.k)


def _gen(key, shape, pos_scale, U, a, R, lr_scale, u_head_div, bf16, nthreads):
    B, H, S, D = shape
    out = np.empty(shape, dtype=np.uint16 if bf16 else np.float32)
    rc = _load().kvpgen_tensor(
        key, B, H, S, D,
        pos_scale.ctypes.data if pos_scale is not None else None,
        U.ctypes.data if U is not None else None,
        a.ctypes.data if a is not None else None,
        R, lr_scale, u_head_div, 1 if bf16 else 0, out.ctypes.data, nthreads)
    if rc != 0:
        raise RuntimeError(f"kvpgen_tensor failed: {rc}")
    return out


def make_layer(wl: Workload, layer: int = 0, nthreads: Optional[int] = None,
               zero_q: bool = False) -> LayerInputs:
    """Generate one layer of workload ``wl`` (shape fields may be overridden
    with ``wl.with_(...)``).  ``zero_q`` replaces Q by zeros (uniform causal
    attention; used for closed-form checks)."""
    if wl.Hq % wl.Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    nthreads = nthreads or default_threads()
    seed = wl.layer_seed(layer)
    bf16 = wl.dtype == "bf16"
    B, Hq, Hkv, S, D = wl.B, wl.Hq, wl.Hkv, wl.S, wl.D
    G = Hq // Hkv

    pos_scale = None
    heavy = np.empty(0, np.int64)
    if S > 0 and (wl.sink_scale != 1.0 or wl.heavy_frac > 0.0):
        pos_scale = np.ones(S, dtype=np.float32)
        n_heavy = int(np.floor(wl.heavy_frac * S)) if S > 1 else 0
        n_heavy = min(n_heavy, max(S - 1, 0))
        if n_heavy:
            heavy = choose(stream_key(seed, TAG_HEAVY), 1, S, n_heavy)
            pos_scale[heavy] = wl.heavy_scale
        pos_scale[0] = wl.sink_scale

    U = a = None
    R = wl.lowrank_rank
    if R:
        U = normals(stream_key(seed, TAG_U), Hkv * D * R).reshape(Hkv, D, R)
        a = normals(stream_key(seed, TAG_A), B * S * R).reshape(B, S, R)

    if zero_q:
        q = np.zeros((B, Hq, S, D), dtype=np.uint16 if bf16 else np.float32)
    else:
        q = _gen(stream_key(seed, TAG_Q), (B, Hq, S, D), None, U, a, R, wl.lowrank_scale,
                 G, bf16, nthreads)
    k = _gen(stream_key(seed, TAG_K), (B, Hkv, S, D), pos_scale, U, a, R, wl.lowrank_scale,
             1, bf16, nthreads)
    return LayerInputs(wl, layer, q, k, heavy)
