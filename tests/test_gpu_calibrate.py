"""The MFMA calibration kernel (a measurement aid, not part of the indexer): its flop count, zero
operands giving zero sums, and one round on random operands matching an fp64 product of the
same operands in the 16x16x32 bf16 MFMA layout (lane l supplies A row l % 16 and B column
l % 16 over k = 8 (l / 16) .. + 7, and receives D rows 4 (l / 16) + r of column l % 16)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_token_idx_amd as m
    assert torch.cuda.is_available()
    return m


def _hash(x):
    x = x.astype(np.uint64) & 0xFFFFFFFF
    x ^= x >> 16
    x = (x * 0x7FEB352D) & 0xFFFFFFFF
    x ^= x >> 15
    x = (x * 0x846CA68B) & 0xFFFFFFFF
    x ^= x >> 16
    return x


def _pair(h):
    lo = (h & 0x80FF) | 0x3F00
    hi = ((h >> 16) & 0x80FF) | 0x3F00
    return lo | (hi << 16)


def _bf16_pairs_to_f64(words):
    """[..., 4] uint32 words of bf16 pairs -> [..., 8] float64 (low half first)."""
    w = words.astype(np.uint64)
    halves = np.stack([w & 0xFFFF, w >> 16], axis=-1).reshape(*w.shape[:-1], 8)
    return (halves.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _emulate_one_round(n_threads):
    ids = np.arange(n_threads, dtype=np.uint64)
    j = np.arange(4, dtype=np.uint64)
    r = np.arange(4, dtype=np.uint64)
    h = _hash(ids[:, None, None] * 64 + 8 * j[None, :, None] + r[None, None, :])   # [n, j, r]
    g = _hash(h ^ 0x9E3779B9)
    a = _bf16_pairs_to_f64(_pair(h))          # [n, 4 (j), 8 (k within the lane's block)]
    b = _bf16_pairs_to_f64(_pair(g))
    W = n_threads // 64
    a = a.reshape(W, 4, 16, 4, 8)             # [wave, l // 16, l % 16, j, k]
    b = b.reshape(W, 4, 16, 4, 8)
    A = a.transpose(0, 3, 2, 1, 4).reshape(W, 4, 16, 32)    # [wave, j, m, k]
    B = b.transpose(0, 3, 1, 4, 2).reshape(W, 4, 32, 16)    # [wave, j, k, n]
    sums = np.zeros((W, 64))
    bound = np.zeros((W, 64))
    for i in range(16):
        D = A[:, i & 3] @ B[:, i >> 2]                       # [wave, 16 (m), 16 (n)]
        Dabs = np.abs(A[:, i & 3]) @ np.abs(B[:, i >> 2])
        for lg in range(4):
            sums[:, 16 * lg:16 * lg + 16] += D[:, 4 * lg:4 * lg + 4, :].sum(axis=1)
            bound[:, 16 * lg:16 * lg + 16] += Dabs[:, 4 * lg:4 * lg + 4, :].sum(axis=1)
    return sums.reshape(-1), bound.reshape(-1)


def test_flop_count_and_zero_operands(dsa):
    flop, sink = dsa.mfma_calibrate(3, random_operands=False)
    torch.cuda.synchronize()
    assert flop == 1024 * 4 * 3 * 16 * 2 * 16 * 16 * 32
    assert torch.count_nonzero(sink).item() == 0


def test_one_round_matches_fp64_products(dsa):
    _, sink = dsa.mfma_calibrate(1, random_operands=True)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().astype(np.float64)
    want, bound = _emulate_one_round(got.size)
    # fp32 accumulation of 32-term products and of the lane's 64 outputs: far inside 2^-18
    assert np.all(np.abs(got - want) <= 2.0 ** -18 * bound), float(np.max(np.abs(got - want) / bound))


def test_repeatable(dsa):
    _, s1 = dsa.mfma_calibrate(50, random_operands=True)
    s1 = s1.clone()
    _, s2 = dsa.mfma_calibrate(50, random_operands=True)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert torch.isfinite(s1).all()
