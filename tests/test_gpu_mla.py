"""GPU parity of the sparse MLA consumer against the CPU oracle: the attention of each query's
96 heads over the latent-cache rows its indexer selected ("Qwen3.5-397B-A17B vs Kimi K3.1
Pro" page, gated-MLA row; absorbed-query reading, as the oracle).

Tolerance, per output element, from the arithmetic the library states (fp32 logits and sums, the
probabilities rounded to bf16 for the weighted sum, and with S > 1 splits of the selection list
into blocks of `per` entries, each split's normalised output rounded to bf16 before the merge),
with p_j the exact probabilities and v_j the value rows:
  * bf16 rounding of p (relative error uniform in +-2^-9, independent): 10 standard deviations,
    10 * 2^-9 / sqrt(3) * sqrt(sum_j p_j^2 v_j^2);
  * bf16 rounding of each split's output: 2^-9 * sum_s |sum_{j in s} p_j v_j|;
  * fp32 logits and exponentials (a relative error rho in each p_j, rho from the accumulation
    radius of the 576-term logit and a few ulps of exp2 and the sums): 2 rho sum_j p_j |v_j|;
  * the final rounding: one bf16 ulp of the exact value.
lse within 1e-4 (1 + |lse|)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import MLA_KV, MLA_V
from synth import workloads as wl
from tests.helpers import bf16_ulp, to_dev, to_host

pytestmark = pytest.mark.gpu
NH = 96


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_token_idx_amd as m
    assert torch.cuda.is_available()
    return m


def _bf(x):
    return oracle.f64_to_bf16(np.asarray(x, dtype=np.float64))


def _case(rng, T, N, topk, qs=0.5, frac_empty=0.0):
    q = _bf(rng.standard_normal((T, NH, MLA_KV)) * qs)
    kv = _bf(rng.standard_normal((N, MLA_KV)))
    idx = np.stack([rng.choice(N, topk, replace=False) for _ in range(T)]).astype(np.int32)
    if frac_empty:
        idx[rng.random(idx.shape) < frac_empty] = -1
    return q, kv, idx


def _splits(dsa, T, topk):
    """(number of splits, selections per split) of a launch, from its workspace size."""
    ws = dsa.workspace_size(dsa.OP_SPARSE_MLA, T, 0, 0, topk)
    S = ws // (T * NH * (2 * MLA_V + 8)) if ws else 1
    per = -(-(-(-topk // S)) // 32) * 32
    return S, per


def _check(dsa, o_gpu, lse_gpu, q, kv, idx, row0=None, scale=192.0 ** -0.5, launch=None):
    T, topk = idx.shape
    S, per = _splits(dsa, *(launch or (T, topk)))
    o_ref, lse_ref = oracle.sparse_mla(q, kv, idx, row0=row0, scale=scale)
    g = oracle.bf16_to_f64(o_gpu)
    kvf = oracle.bf16_to_f64(kv)
    base = np.zeros(T, np.int64) if row0 is None else np.asarray(row0)
    u = 2.0 ** -24
    for t in range(T):
        sel = np.nonzero(idx[t] >= 0)[0]
        if len(sel) == 0:
            assert np.all(g[t] == 0) and np.all(np.isneginf(lse_gpu[t])), f"query {t}: empty selection"
            continue
        rows = kvf[idx[t][sel] + base[t]]                       # [n, 576]
        qf = oracle.bf16_to_f64(q[t])                           # [96, 576]
        z = scale * (qf @ rows.T)
        p = np.exp(z - lse_ref[t][:, None])                     # exact probabilities [96, n]
        v = rows[:, :MLA_V]
        # relative error of each p from the fp32 logits (10-sigma accumulation radius) and
        # a few ulps of exp2, the running sum and the reciprocal
        dz = 10 * u * np.sqrt(576 / 3) * np.sqrt((qf * qf) @ (rows * rows).T) * scale
        rho = 2 * dz.max(axis=1, keepdims=True) + 2 * u * np.abs(z).max(axis=1, keepdims=True) + 16 * u
        tol = 10 * 2.0 ** -9 / np.sqrt(3) * np.sqrt((p * p) @ (v * v)) + 2 * rho * (p @ np.abs(v))
        if S > 1:
            part = np.zeros_like(o_ref[t])
            for s0 in range(0, topk, per):
                m = (sel >= s0) & (sel < s0 + per)
                part += np.abs(p[:, m] @ v[m])
            tol += 2.0 ** -9 * part
        tol += bf16_ulp(o_ref[t])
        err = np.abs(g[t] - o_ref[t])
        j = np.unravel_index(np.argmax(err - tol), err.shape)
        assert (err <= tol).all(), f"query {t}: output error {err[j]} at {j} (tolerance {tol[j]}, |o| {abs(o_ref[t][j])})"
        assert np.all(np.abs(lse_gpu[t] - lse_ref[t]) <= 1e-4 * (1 + np.abs(lse_ref[t]))), f"query {t}: lse"


@pytest.mark.parametrize("T,topk", [(5, 100), (3, 2048), (64, 2048), (700, 256), (1, 1), (2, 33)])
def test_sparse_mla_matches_oracle(dsa, T, topk):
    rng = np.random.default_rng(T * 1000 + topk)
    N = max(4 * topk, 3000)
    q, kv, idx = _case(rng, T, N, topk)
    print(f"sparse mla: T={T} topk={topk} splits={dsa.workspace_size(dsa.OP_SPARSE_MLA, T, 0, 0, topk)}",
          flush=True)
    o, lse = dsa.sparse_mla(to_dev(q), to_dev(kv), torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    _check(dsa, to_host(o).reshape(T, NH, MLA_V), lse.cpu().numpy(), q, kv, idx)


@pytest.mark.parametrize("qs", [2.0, 4.0])
def test_sparse_mla_peaked_softmax(dsa, qs):
    """Large logits (std about 3.5 and 7): a few selections carry most of the weight, so each
    output is close to one value row and the tolerance is a small fraction of it."""
    rng = np.random.default_rng(int(qs * 10))
    T, topk = 8, 2048
    q, kv, idx = _case(rng, T, 3 * topk, topk, qs=qs)
    o, lse = dsa.sparse_mla(to_dev(q), to_dev(kv), torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    _check(dsa, to_host(o).reshape(T, NH, MLA_V), lse.cpu().numpy(), q, kv, idx)


def test_sparse_mla_logit_far_above_the_first_tiles(dsa):
    """The kernel weighs each head against a reference taken from its first tile and runs a split
    again when a later logit lies more than 64 (log2 units) above it.  Planted rows give single
    heads a logit about 100 log2 units above the rest: later in a split (the rerun), and in a
    split's first tile (later weights then underflow to 0 against the high reference)."""
    rng = np.random.default_rng(12)
    T, N, topk = 4, 6000, 2048
    q, kv, idx = _case(rng, T, N, topk)
    S, per = _splits(dsa, T, topk)
    assert S > 1
    qf = oracle.bf16_to_f64(q)
    alpha = 100.0 / (np.log2(np.e) * 192.0 ** -0.5)       # scale * alpha * log2(e) = 100
    planted = []
    for t in range(T):
        for i, h in enumerate([0, 17, 50, 95]):
            s = (t + 3 * i) % S
            pos = s * per + (160 + h % 32 if i % 2 == 0 else 3)   # a later tile, or the first
            idx[t, pos] = N + len(planted)                         # a row of its own
            planted.append(alpha * qf[t, h] / (qf[t, h] @ qf[t, h]))
    kv = np.concatenate([kv, _bf(np.asarray(planted))])
    o, lse = dsa.sparse_mla(to_dev(q), to_dev(kv), torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    _check(dsa, to_host(o).reshape(T, NH, MLA_V), lse.cpu().numpy(), q, kv, idx)


def test_sparse_mla_empty_slots_offsets_and_empty_queries(dsa):
    rng = np.random.default_rng(3)
    T, N, topk = 6, 5000, 300
    q, kv, idx = _case(rng, T, N - 1000, topk, frac_empty=0.3)
    idx[2] = -1                                   # a query with no selection at all
    row0 = np.array([0, 17, 1000, 5, 999, 1000], np.int64)
    kv_full = _bf(rng.standard_normal((N, MLA_KV)))
    o, lse = dsa.sparse_mla(to_dev(q), to_dev(kv_full), torch.from_numpy(idx).cuda(),
                            row0=torch.from_numpy(row0).cuda())
    torch.cuda.synchronize()
    _check(dsa, to_host(o).reshape(T, NH, MLA_V), lse.cpu().numpy(), q, kv_full, idx, row0=row0)


def test_sparse_mla_single_selection_is_exact(dsa):
    rng = np.random.default_rng(4)
    T, N = 4, 700
    q, kv, _ = _case(rng, T, N, 1)
    idx = np.full((T, 40), -1, np.int32)
    idx[np.arange(T), [0, 13, 31, 39]] = [5, 600, 0, 699]
    o, lse = dsa.sparse_mla(to_dev(q), to_dev(kv), torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    o = to_host(o).reshape(T, NH, MLA_V)
    for t, r in enumerate([5, 600, 0, 699]):
        assert np.array_equal(o[t], np.broadcast_to(kv[r, :MLA_V], (NH, MLA_V)))


def test_sparse_mla_on_the_decode_selection(dsa):
    # the consumer step: the indexer's decode selection (indices relative to each sequence's
    # cache start) drives the attention over a latent cache laid out like the key cache
    lens = [3000, 20000, 40000, 2500]
    B = len(lens)
    cache, start = wl.decode_cache(np.asarray(lens), seed=21)
    rng = np.random.default_rng(21)
    qi = _bf(rng.standard_normal((B, 32, 128)))
    wi = _bf(rng.standard_normal((B, 32)) * 0.3)
    idx, _ = dsa.decode(to_dev(qi), to_dev(wi), to_dev(cache), torch.from_numpy(start).cuda(),
                        torch.from_numpy(np.asarray(lens, np.int32)).cuda(), max(lens), topk=2048)
    latent = _bf(rng.standard_normal((sum(lens), MLA_KV)))
    qm = _bf(rng.standard_normal((B, NH, MLA_KV)) * 0.5)
    o, lse = dsa.sparse_mla(to_dev(qm), to_dev(latent), idx, row0=torch.from_numpy(start).cuda())
    torch.cuda.synchronize()
    _check(dsa, to_host(o).reshape(B, NH, MLA_V), lse.cpu().numpy(), qm, latent, idx.cpu().numpy(),
           row0=start)


def test_sparse_mla_full_decode_size(dsa):
    # the benchmark's launch: 64 queries, top 2,048 each, over a latent cache with one row per
    # cached token of the decode workload (5.2M rows); sampled queries against the oracle,
    # which gets only their selected rows
    lens = wl.decode_lengths(64, seed=0)
    cache, start = wl.decode_cache(lens, seed=0)
    B = len(lens)
    rng = np.random.default_rng(64)
    qi = _bf(rng.standard_normal((B, 32, 128)))
    wi = _bf(rng.standard_normal((B, 32)) * 0.3)
    print(f"sparse mla full size: B={B}, {int(lens.sum())} cache rows", flush=True)
    idx, _ = dsa.decode(to_dev(qi), to_dev(wi), to_dev(cache), torch.from_numpy(start).cuda(),
                        torch.from_numpy(lens.astype(np.int32)).cuda(), int(lens.max()), topk=2048)
    del cache
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    latent = torch.empty((int(lens.sum()), MLA_KV), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, latent.shape[0], 1 << 20):
        r1 = min(latent.shape[0], r0 + (1 << 20))
        latent[r0:r1] = torch.randn((r1 - r0, MLA_KV), generator=g, device="cuda").to(torch.bfloat16)
    qm = _bf(rng.standard_normal((B, NH, MLA_KV)) * 0.5)
    start_d = torch.from_numpy(start).cuda()
    o, lse = dsa.sparse_mla(to_dev(qm), latent, idx, row0=start_d)
    torch.cuda.synchronize()
    assert dsa.workspace_size(dsa.OP_SPARSE_MLA, B, 0, 0, 2048) > 0   # the split launch
    pick = np.array([0, 9, 17, 31, 40, 52, 60, 63])
    idx_h = idx.cpu().numpy()[pick]
    rows = torch.from_numpy((idx_h.astype(np.int64) + start[pick, None]).reshape(-1)).cuda()
    kv_sel = to_host(latent[rows])                        # the sampled queries' rows, in order
    local = np.where(idx_h >= 0, np.arange(len(pick) * 2048, dtype=np.int32).reshape(len(pick), 2048), -1)
    _check(dsa, to_host(o).reshape(B, NH, MLA_V)[pick], lse.cpu().numpy()[pick], qm[pick], kv_sel, local,
           launch=(B, 2048))
