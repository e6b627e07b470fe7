"""GPU parity of the decode paths that the common workload does not reach: a row whose sampled
threshold overshoots (re-scored in full by its select workgroup), rows of equal scores (all
scores written and selected from), very large batches (the prefix pass) and long rows split
into many pieces; bf16 and FP8 caches.  Every case is checked against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from oracle import D, H
from synth import workloads as wl
from tests.helpers import check_row, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_token_idx_amd as m
    assert torch.cuda.is_available()
    return m


def _bf(x):
    return oracle.f64_to_bf16(np.asarray(x, dtype=np.float64))


def _sample_positions(b, n):
    """The plan pass's sample of row b (n keys): S = 2^lgS >= n / 128 keys (1,024 .. 8,192) in
    S / 8 runs of 8 consecutive keys; run j lies in stratum j of S / 8 at an offset that is an
    integer hash of (b, j) scaled to the stratum width less 8."""
    lgS = 10
    while lgS < 13 and (1 << lgS) < n // 128:
        lgS += 1
    S = 1 << lgS
    M = 0xFFFFFFFF
    pos = []
    for i in range(S):
        j = i >> 3
        lo, hi = (j * n) >> (lgS - 3), ((j + 1) * n) >> (lgS - 3)
        x = (j + 0x9E3779B9 * (b + 1)) & M
        x ^= x >> 16
        x = (x * 0x7FEB352D) & M
        x ^= x >> 15
        x = (x * 0x846CA68B) & M
        x ^= x >> 16
        pos.append(lo + ((x * (hi - lo - 7)) >> 32) + (i & 7))
    return np.asarray(pos)


def _run(dsa, q, w, cache, start, lens, topk, fp8):
    lens_d = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    start_d = torch.from_numpy(np.asarray(start, np.int64)).cuda()
    if fp8:
        k8, sc = dsa.quantize_keys(to_dev(cache))
        idx, s = dsa.decode_fp8(to_dev(q), to_dev(w), k8, sc, start_d, lens_d, max(lens), topk=topk)
    else:
        idx, s = dsa.decode(to_dev(q), to_dev(w), to_dev(cache), start_d, lens_d, max(lens), topk=topk)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), s.cpu().numpy()


def _oracle(q, w, cache, start, lens, rows, topk, fp8):
    rows = np.asarray(rows)
    t = np.asarray(lens)[rows] - 1
    if fp8:
        codes, exps = oracle.quantize_e4m3(cache)
        return oracle.rows_fp8(q[rows], w[rows], codes, exps, np.asarray(start)[rows], t, topk=topk, full=True)
    return oracle.rows(q[rows], w[rows], cache, np.asarray(start)[rows], t, topk=topk, full=True)


@pytest.mark.parametrize("fp8", [False, True])
def test_sample_overshoot_is_rescored(dsa, fp8):
    # The keys the plan pass samples in row 1 get scores far above every other key (distinct
    # up to bf16 rounding), so its threshold lets through fewer than topk candidates: the
    # select workgroup must score the row again and still return the exact top-k.
    rng = np.random.default_rng(7)
    lens = [20000, 40000, 30000]
    B = len(lens)
    start = np.concatenate([[0], np.cumsum(lens)[:-1]])
    q = _bf(rng.standard_normal((B, H, D)))
    w = _bf(np.abs(rng.standard_normal((B, H))) * 0.3)
    kf = rng.standard_normal((sum(lens), D))
    b = 1
    hot = oracle.bf16_to_f64(q[b]).sum(axis=0)
    hot = 3.0 * hot / np.abs(hot).max()
    pos = _sample_positions(b, lens[b])
    kf[start[b] + pos] = hot[None, :] * (1.0 + np.arange(len(pos))[:, None] / 512.0)
    cache = _bf(kf)
    print(f"overshoot: fp8={fp8}, {len(pos)} hot sampled keys in row {b}", flush=True)
    idx, sc = _run(dsa, q, w, cache, start, lens, 2048, fp8)
    ref = _oracle(q, w, cache, start, lens, range(B), 2048, fp8)
    for r in range(B):
        check_row(lens[r] - 1, idx[r], sc[r], ref, r, 2048)
    # the hot keys are among the winners of row b
    assert set((pos[:256]).tolist()) <= set(idx[b].tolist())


@pytest.mark.parametrize("fp8", [False, True])
def test_equal_scores_take_the_lowest_indices(dsa, fp8):
    # w = 0: every score is 0; long rows are planned dense (all scores written)
    rng = np.random.default_rng(8)
    lens = [50000, 17000, 3000]
    B = len(lens)
    start = np.concatenate([[0], np.cumsum(lens)[:-1]])
    q = _bf(rng.standard_normal((B, H, D)))
    w = np.zeros((B, H), np.uint16)
    cache = _bf(rng.standard_normal((sum(lens), D)))
    idx, sc = _run(dsa, q, w, cache, start, lens, 2048, fp8)
    assert np.array_equal(idx, np.broadcast_to(np.arange(2048, dtype=np.int32), idx.shape))
    assert np.all(sc == 0)


@pytest.mark.parametrize("fp8", [False, True])
def test_many_sequences_prefix_pass(dsa, fp8):
    # more sequences than the plan pass sums itself: the separate prefix pass
    B = 5000
    lens = (np.random.default_rng(9).integers(1, 120, B)).tolist()
    start = np.concatenate([[0], np.cumsum(lens)[:-1]])
    rng = np.random.default_rng(10)
    q = _bf(rng.standard_normal((B, H, D)))
    w = _bf(rng.standard_normal((B, H)) * 0.3)
    cache = _bf(rng.standard_normal((sum(lens), D)))
    idx, sc = _run(dsa, q, w, cache, start, lens, 16, fp8)
    rows = [0, 1, 2, 777, 2500, 4998, 4999]
    ref = _oracle(q, w, cache, start, lens, rows, 16, fp8)
    for j, r in enumerate(rows):
        check_row(lens[r] - 1, idx[r], sc[r], ref, j, 16)


@pytest.mark.parametrize("fp8", [False, True])
def test_long_row_many_pieces(dsa, fp8):
    # one row far longer than the others: split over thousands of filter waves
    lens = [300000, 40000, 100, 70001]
    B = len(lens)
    cache, start = wl.decode_cache(np.asarray(lens), seed=12)
    rng = np.random.default_rng(12)
    q = _bf(rng.standard_normal((B, H, D)))
    w = _bf(rng.standard_normal((B, H)) * 0.3)
    idx, sc = _run(dsa, q, w, cache, start, lens, 2048, fp8)
    ref = _oracle(q, w, cache, start, lens, range(B), 2048, fp8)
    for r in range(B):
        check_row(lens[r] - 1, idx[r], sc[r], ref, r, 2048)
