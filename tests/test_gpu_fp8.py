"""GPU parity of the FP8 (OCP E4M3) key-cache path against the CPU oracle: cache
quantisation bit for bit, and decode against an FP8 cache within the score tolerance."""
import numpy as np
import pytest
import torch

import oracle
from oracle import D, H
from synth import workloads as wl
from tests.helpers import check_row, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_token_idx_amd as m
    assert torch.cuda.is_available()
    return m


def _bf(x):
    return oracle.f64_to_bf16(np.asarray(x, dtype=np.float64))


def _keys(n, seed):
    rng = np.random.default_rng(seed)
    mag = 10.0 ** rng.uniform(-6, 6, (n, 1))
    return _bf(rng.standard_normal((n, D)) * mag)


def test_quantize_keys_bit_exact(dsa):
    k = _keys(1000, seed=1)
    k[3] = 0                                    # all zeros: scale 1, codes 0
    k[4] = 0x8000                               # all -0: codes 0x80
    k[5, :] = 0
    k[5, 7] = _bf([-3.0])[0]                    # one nonzero
    k[6] = _bf(np.linspace(-448, 448, D))       # the edge of the E4M3 range at scale 1
    k8, sc = dsa.quantize_keys(to_dev(k))
    torch.cuda.synchronize()
    codes, exps = oracle.quantize_e4m3(k)
    assert np.array_equal(k8.cpu().numpy(), codes)
    assert np.array_equal(sc.cpu().numpy(), (2.0 ** exps).astype(np.float32))


def test_quantize_keys_slots_and_stride(dsa):
    k = _keys(300, seed=2)
    wide = torch.zeros((300, 256), dtype=torch.bfloat16, device="cuda")
    wide[:, :D] = to_dev(k)
    slots = np.random.default_rng(3).permutation(500)[:300].astype(np.int64)
    k8 = torch.zeros((500, D), dtype=torch.uint8, device="cuda")
    sc = torch.zeros((500,), dtype=torch.float32, device="cuda")
    dsa.quantize_keys(wide[:, :D], k8, sc, slot=torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    codes, exps = oracle.quantize_e4m3(k)
    assert np.array_equal(k8.cpu().numpy()[slots], codes)
    assert np.array_equal(sc.cpu().numpy()[slots], (2.0 ** exps).astype(np.float32))
    rest = np.setdiff1d(np.arange(500), slots)
    assert np.all(k8.cpu().numpy()[rest] == 0) and np.all(sc.cpu().numpy()[rest] == 0)


def _fp8_case(dsa, lens, seed, topk=2048):
    rng = np.random.default_rng(seed)
    B = len(lens)
    q = _bf(rng.standard_normal((B, H, D)))
    w = _bf(rng.standard_normal((B, H)) * 0.3)
    cache, start = wl.decode_cache(np.asarray(lens), seed=seed)
    k8, sc = dsa.quantize_keys(to_dev(cache))
    idx, scores = dsa.decode_fp8(to_dev(q), to_dev(w), k8, sc, torch.from_numpy(start).cuda(),
                                 torch.from_numpy(np.asarray(lens, np.int32)).cuda(), max(lens),
                                 topk=topk)
    torch.cuda.synchronize()
    codes, exps = oracle.quantize_e4m3(cache)
    assert np.array_equal(k8.cpu().numpy(), codes)
    return dict(q=q, w=w, codes=codes, exps=exps, start=start, idx=idx.cpu().numpy(),
                sc=scores.cpu().numpy())


def test_decode_fp8_small(dsa):
    lens = [1, 2, 100, 2048, 2049, 5000, 4097, 16385, 20001]
    r = _fp8_case(dsa, lens, seed=5)
    ref = oracle.rows_fp8(r["q"], r["w"], r["codes"], r["exps"], r["start"], np.asarray(lens) - 1,
                          topk=2048, full=True)
    for b, L in enumerate(lens):
        check_row(L - 1, r["idx"][b], r["sc"][b], ref, b, 2048)


@pytest.mark.parametrize("topk", [1, 5, 100])
def test_decode_fp8_small_topk(dsa, topk):
    lens = [1, 50, 3000, 17000]
    r = _fp8_case(dsa, lens, seed=10 + topk, topk=topk)
    ref = oracle.rows_fp8(r["q"], r["w"], r["codes"], r["exps"], r["start"], np.asarray(lens) - 1,
                          topk=topk, full=True)
    for b, L in enumerate(lens):
        check_row(L - 1, r["idx"][b], r["sc"][b], ref, b, topk)


def test_decode_fp8_64_sequences(dsa):
    # the decode workload: 64 sequences with U[32768, 131072] cached keys, sampled rows checked
    lens = wl.decode_lengths(64, seed=0)
    print(f"decode fp8: B=64, {int(lens.sum())} cached keys", flush=True)
    r = _fp8_case(dsa, lens.tolist(), seed=0)
    sample = np.array([0, 1, int(np.argmax(lens)), int(np.argmin(lens)), 31, 63])
    ref = oracle.rows_fp8(r["q"][sample], r["w"][sample], r["codes"], r["exps"], r["start"][sample],
                          lens[sample] - 1, topk=2048, full=True)
    for j, b in enumerate(sample):
        check_row(int(lens[b]) - 1, r["idx"][b], r["sc"][b], ref, j, 2048)
