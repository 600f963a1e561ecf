"""kvp_select_topk_noalloc, called through the C ABI: the keep-set selection
for callers that cannot allocate, whose split-path state lives in the
library's own per-GPU device array.  Its output must equal that of
kvp_select_topk (with a caller workspace) bit for bit -- and hence the
oracle's selection, which the other select tests compare kvp_select_topk
with -- on two calls in a row, the second with a smaller input, so the
array's leftovers from the first call must not matter."""
import ctypes

import numpy as np
import pytest
import torch

import future_attention_scoring_kvp_amd as kvp
import oracle
from parity import say

pytestmark = pytest.mark.gpu

OK, WORKSPACE = 0, 3
MAX_BYTES = 32 << 20


@pytest.fixture(scope="module")
def lib():
    lib = kvp.load_library()
    lib.kvp_select_topk_noalloc.restype = ctypes.c_int
    lib.kvp_select_topk_noalloc.argtypes = [ctypes.c_void_p, kvp._Dims, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.c_void_p]
    return lib


def noalloc(lib, m, w, s, k):
    rows, S = m.shape[0] * m.shape[1], m.shape[2]
    keep = torch.full((rows, kvp.keep_count(S, w, s, k)), -7, dtype=torch.int32, device="cuda")
    st = lib.kvp_select_topk_noalloc(m.data_ptr(), kvp._Dims(rows, 1, 1, S, 128), w, s, k,
                                     keep.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == OK, st
    torch.cuda.synchronize()
    return keep.view(m.shape[0], m.shape[1], -1).cpu().numpy()


def test_noalloc_matches_workspace_select_on_two_calls(lib):
    rng = np.random.default_rng(20261203)
    cases = [
        # 8 KV heads of one 128K-token layer, k = 2048 (split path, 32 chunks per row)
        ((1, 8, 131072), 1024, 4, 2048, "mass"),
        # a smaller second call: 3 rows of 40001 with long runs of ties
        ((1, 3, 40001), 300, 4, 5000, "ties"),
    ]
    for (B, H, S), w, s, k, kind in cases:
        if kind == "mass":
            m = (rng.standard_normal((B, H, S)) ** 2).astype(np.float32)
        else:
            m = (np.round(rng.standard_normal((B, H, S)) * 40) / 8).astype(np.float32)
        assert kvp.select_workspace_bytes(B * H, S, k) <= MAX_BYTES
        dev = torch.from_numpy(m).cuda()
        say(f"[noalloc] {B}x{H}x{S} w={w} s={s} k={k}")
        got = noalloc(lib, dev, w, s, k)
        ref = kvp.select_topk(dev, w, s, k).cpu().numpy()
        assert np.array_equal(got, ref), f"{B}x{H}x{S}: differs from kvp_select_topk"
        exact = oracle.select(m.astype(np.float64), w, s, k)
        assert np.array_equal(got, exact), f"{B}x{H}x{S}: differs from the oracle"


def test_noalloc_short_rows_and_limit(lib):
    rng = np.random.default_rng(4)
    m = torch.from_numpy(rng.standard_normal((2, 8, 4096)).astype(np.float32)).cuda()
    got = noalloc(lib, m, 128, 4, 512)   # register path: the array is not used
    assert np.array_equal(got, kvp.select_topk(m, 128, 4, 512).cpu().numpy())
    # more rows than the array holds: rejected before any launch
    S = 1 << 22
    rows = 4
    assert kvp.select_workspace_bytes(rows, S, 10) > MAX_BYTES
    st = lib.kvp_select_topk_noalloc(0x100000, kvp._Dims(rows, 1, 1, S, 128), 16, 4, 10,
                                     0x100000, None)
    assert st == WORKSPACE
