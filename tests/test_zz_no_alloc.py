"""The decode entry that allocates nothing (dsa_idx_decode_noalloc, its scratch a static device
array) against dsa_idx_decode with a caller workspace: the same kernels, so the same indices and
scores bit for bit, on two calls in a row, the second smaller than the first (the array keeps
the first call's contents).  Also: a request larger than the array is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from synth import workloads as wl
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_token_idx_amd as m
    assert torch.cuda.is_available()
    return m


def _case(B, lo, hi, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, B).astype(np.int64)
    cache, start = wl.decode_cache(lens, seed=seed)
    q = (rng.standard_normal((B, 32, 128))).astype(np.float32)
    w = (rng.standard_normal((B, 32)) * 0.3).astype(np.float32)
    return (torch.from_numpy(q).to(torch.bfloat16).cuda(), torch.from_numpy(w).to(torch.bfloat16).cuda(),
            to_dev(cache), torch.from_numpy(start).cuda(), torch.from_numpy(lens.astype(np.int32)).cuda(),
            int(lens.max()))


def _noalloc(dsa, q, w, cache, start, lens, maxL, topk):
    B = q.shape[0]
    idx = torch.empty((B, topk), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, topk), dtype=torch.float32, device="cuda")
    vp = ctypes.c_void_p
    rc = dsa.lib().dsa_idx_decode_noalloc(vp(q.data_ptr()), vp(w.data_ptr()), vp(cache.data_ptr()),
                                          vp(start.data_ptr()), vp(lens.data_ptr()), B, maxL, topk,
                                          vp(idx.data_ptr()), vp(sc.data_ptr()),
                                          vp(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, dsa.lib().dsa_idx_last_error()
    return idx, sc


def test_noalloc_decode_matches_decode_on_two_calls(dsa):
    for B, lo, hi, seed, topk in ((24, 20000, 90000, 1, 2048), (5, 1, 30000, 2, 100)):
        print(f"no-alloc decode: B={B}, lengths {lo}..{hi}, topk {topk}", flush=True)
        q, w, cache, start, lens, maxL = _case(B, lo, hi, seed)
        ref_i, ref_s = dsa.decode(q, w, cache, start, lens, maxL, topk=topk)
        got_i, got_s = _noalloc(dsa, q, w, cache, start, lens, maxL, topk)
        torch.cuda.synchronize()
        assert torch.equal(got_i, ref_i)
        assert torch.equal(got_s.view(torch.int32), ref_s.view(torch.int32))


def test_noalloc_decode_refuses_oversized_requests(dsa):
    L = dsa.lib()
    vp = ctypes.c_void_p
    A = 0x10000
    rc = L.dsa_idx_decode_noalloc(vp(A), vp(A), vp(A), vp(A), vp(A), 4096, 131072, 2048, vp(A), None, None)
    assert rc == -2 and b"scratch" in L.dsa_idx_last_error()
    assert L.dsa_idx_decode_noalloc(None, None, None, None, None, 0, 0, 8, None, None, None) == 0
