"""GPU parity of the 64-head (DeepSeek-V3.2-shaped) indexer against the CPU oracle.

Projections: q, k and w against the exact fp64 products (the accumulation radius of linear_exact
in tests/helpers.py), with the rotary step applied to the exact values; the library rotates the
fp32 results in its projection epilogues and rounds once, so each rotated element must be the
bf16 rounding of a value within the rotated radius.  Scores and selection: the parity rule of
tests/helpers.py, with the oracle scoring all 64 heads."""
import numpy as np
import pytest
import torch

import oracle
from oracle import D, V32_H
from synth import workloads as wl
from tests.helpers import (U32, check_projection, check_row, layernorm_exact, linear_exact, to_dev, to_host,
                           weights_to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_token_idx_amd as m
    assert torch.cuda.is_available()
    return m


def _rot_radius(exact, r, pos):
    """(exact rotated values, radius of the GPU's fp32 rotated values around them): the rotation
    carries the accumulation error vector of a pair unchanged in length, and the fp32 rotation
    (products, fma, cos and sin rounded to fp32) adds at most 6 u of the pair's length."""
    rot = oracle.rope_f64(exact, pos)
    out = r.copy()
    pr = np.sqrt(r[..., 0:64:2] ** 2 + r[..., 1:64:2] ** 2) \
        + 6 * U32 * np.sqrt(exact[..., 0:64:2] ** 2 + exact[..., 1:64:2] ** 2)
    out[..., 0:64:2] = pr
    out[..., 1:64:2] = pr
    return rot, out


@pytest.mark.parametrize("T,pos0", [(1, 0), (37, 5000), (300, 0), (130, 1_000_000)])
def test_v32_project_matches_oracle(dsa, T, pos0):
    Wt = wl.layer_weights_v32(seed=T)
    act = wl.layer_activations(T, seed=T + 1)
    print(f"v32 project: T={T} pos0={pos0}", flush=True)
    q, k, w = dsa.v32_project(to_dev(act["x"]), to_dev(act["c_q"]), weights_to_dev(Wt), pos0=pos0)
    torch.cuda.synchronize()
    pos = pos0 + np.arange(T)
    # each element: the bf16 rounding of an fp32 value within the rotated accumulation radius of
    # the exact rotated projection
    eq, rq = linear_exact(act["c_q"], Wt["W_q"])
    eq, rq = eq.reshape(T, V32_H, D), rq.reshape(T, V32_H, D)
    check_projection(to_host(q).reshape(T, V32_H, D), *_rot_radius(eq, rq, pos), "q")
    check_projection(to_host(w), *linear_exact(act["x"], Wt["W_w"]), "w")
    ek, rk = layernorm_exact(*linear_exact(act["x"], Wt["W_k"]), Wt)
    check_projection(to_host(k), *_rot_radius(ek, rk, pos), "k")
    # and nearly always the oracle's own bf16 values
    oq, ok, ow = oracle.project_v32(act["x"], act["c_q"], Wt, pos0=pos0)
    fr = [float((to_host(g).reshape(o.shape) != o).mean()) for g, o in ((q, oq), (k, ok), (w, ow))]
    print(f"  fraction differing from the oracle's bf16 values: q {fr[0]:.1e} k {fr[1]:.1e} w {fr[2]:.1e}")
    assert max(fr) < 2e-2


def _inputs(T, seed):
    rng = np.random.default_rng(seed)
    q = oracle.f64_to_bf16(rng.standard_normal((T, V32_H, D)))
    k = oracle.f64_to_bf16(rng.standard_normal((T, D)))
    w = oracle.f64_to_bf16(rng.standard_normal((T, V32_H)) * np.sqrt(0.1))
    return q, k, w


@pytest.mark.parametrize("T,topk", [(1, 5), (300, 2048), (2600, 2048), (2600, 100)])
def test_v32_score_topk_matches_oracle(dsa, T, topk):
    q, k, w = _inputs(T, T + topk)
    print(f"v32 score_topk: T={T} topk={topk}", flush=True)
    idx, sc = dsa.v32_score_topk(to_dev(q), to_dev(k), to_dev(w), topk=topk)
    torch.cuda.synchronize()
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    rows = np.arange(T) if T <= 300 else np.array([0, 1, 127, 128, 129, 1000, 2047, 2048, 2049, 2599])
    ref = oracle.prefill_rows(q, k, w, rows, topk=topk, full=True)
    for r, t in enumerate(rows):
        check_row(int(t), idx[t], sc[t], ref, r, topk)


def test_v32_end_to_end(dsa):
    T = 700
    Wt = wl.layer_weights_v32(seed=11)
    act = wl.layer_activations(T, seed=11)
    print(f"v32 end to end: T={T}", flush=True)
    q, k, w = dsa.v32_project(to_dev(act["x"]), to_dev(act["c_q"]), weights_to_dev(Wt))
    idx, sc = dsa.v32_score_topk(q, k, w, topk=256)
    torch.cuda.synchronize()
    qh, kh, wh = to_host(q).reshape(T, V32_H, D), to_host(k), to_host(w)
    rows = np.array([0, 255, 256, 257, 511, 699])
    ref = oracle.prefill_rows(qh, kh, wh, rows, topk=256, full=True)
    for r, t in enumerate(rows):
        check_row(int(t), idx.cpu().numpy()[t], sc.cpu().numpy()[t], ref, r, 256)


def test_v32_full_size_sampled_rows(dsa):
    # the benchmark's launch: T = 65,536, top 2,048, checked on sampled rows
    T, topk = 65536, 2048
    q, k, w = _inputs(T, 7)
    print(f"v32 full size: T={T}", flush=True)
    idx, sc = dsa.v32_score_topk(to_dev(q), to_dev(k), to_dev(w), topk=topk)
    torch.cuda.synchronize()
    rows = np.array([0, 2047, 2048, 30000, 65535])
    idx, sc = idx[rows].cpu().numpy(), sc[rows].cpu().numpy()
    ref = oracle.prefill_rows(q, k, w, rows, topk=topk, full=True)
    for r, t in enumerate(rows):
        check_row(int(t), idx[r], sc[r], ref, r, topk)


def test_v32_varlen_equals_per_sequence(dsa):
    lens = [1, 130, 2049, 700, 2048]
    total = sum(lens)
    q, k, w = _inputs(total, 21)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    print(f"v32 varlen: lens={lens}", flush=True)
    qd, kd, wd = to_dev(q), to_dev(k), to_dev(w)
    idx, sc = dsa.v32_score_topk_varlen(qd, kd, wd, torch.from_numpy(cu).cuda(), max(lens), topk=256)
    torch.cuda.synchronize()
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    for b, L in enumerate(lens):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        i1, c1 = dsa.v32_score_topk(qd[s0:s1].contiguous(), kd[s0:s1].contiguous(), wd[s0:s1].contiguous(),
                                    topk=256)
        assert np.array_equal(idx[s0:s1], i1.cpu().numpy()), f"sequence {b}: indices differ"
        assert np.array_equal(sc[s0:s1].view(np.uint32), c1.cpu().numpy().view(np.uint32)), f"sequence {b}: scores differ"
        rows = np.unique(np.array([0, L // 2, L - 1]))
        ref = oracle.prefill_rows(q[s0:s1], k[s0:s1], w[s0:s1], rows, topk=256, full=True)
        for r, t in enumerate(rows):
            check_row(int(t), idx[s0 + t], sc[s0 + t], ref, r, 256)


def test_v32_chunk_equals_the_last_rows(dsa):
    # C queries at offset prefix against the whole prefix: the last C rows of the one-sequence
    # call, bit for bit (offsets inside and across 128-key tiles)
    T, topk = 2600, 512
    q, k, w = _inputs(T, 31)
    qd, kd, wd = to_dev(q), to_dev(k), to_dev(w)
    full_i, full_s = dsa.v32_score_topk(qd, kd, wd, topk=topk)
    for prefix in (0, 77, 2048, 2500):
        C = T - prefix
        print(f"v32 chunk: prefix={prefix} C={C}", flush=True)
        ci, cs = dsa.prefill_chunk(qd[prefix:].contiguous(), kd, wd[prefix:].contiguous(), prefix, topk=topk)
        torch.cuda.synchronize()
        assert torch.equal(ci, full_i[prefix:]), f"prefix {prefix}: indices differ"
        assert torch.equal(cs.view(torch.int32), full_s[prefix:].view(torch.int32)), f"prefix {prefix}: scores differ"


@pytest.mark.parametrize("topk", [2048, 100])
def test_v32_decode(dsa, topk):
    # one new query per sequence against its cached keys, the new token's key written by the
    # 64-head projection at its own position; stage-wise against the oracle on the GPU's own
    # projections and cache, and equal to the last row of the one-sequence call
    lens = [1, 100, 2048, 2049, 5000, 40000]
    B = len(lens)
    Wt = wl.layer_weights_v32(seed=41)
    act = wl.layer_activations(B, seed=41)
    cache, start = wl.decode_cache(np.asarray(lens), seed=41)
    cache_d = to_dev(cache)
    Wd = weights_to_dev(Wt)
    print(f"v32 decode: lens={lens} topk={topk}", flush=True)
    qs, ws_ = [], []
    for b, L in enumerate(lens):   # each token at its own position L - 1
        q1, k1, w1 = dsa.v32_project(to_dev(act["x"][b:b + 1]), to_dev(act["c_q"][b:b + 1]), Wd, pos0=L - 1)
        cache_d[start[b] + L - 1] = k1[0]
        qs.append(q1)
        ws_.append(w1)
    q = torch.cat(qs)
    w = torch.cat(ws_)
    idx, sc = dsa.decode(q, w, cache_d, torch.from_numpy(start).cuda(),
                         torch.from_numpy(np.asarray(lens, np.int32)).cuda(), max(lens), topk=topk)
    torch.cuda.synchronize()
    qh, wh, ch = to_host(q).reshape(B, V32_H, D), to_host(w), to_host(cache_d)
    ref = oracle.rows(qh, wh, ch, start, np.asarray(lens) - 1, topk=topk, full=True)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    for b, L in enumerate(lens):
        check_row(L - 1, idx[b], sc[b], ref, b, topk)


def test_v32_decode_fp8(dsa):
    # the 64-head decode against the FP8 key cache: stage-wise against the oracle's FP8 rows
    # (queries quantised per head there too) on the GPU's own projections and cache codes
    lens = [1, 300, 2049, 9000]
    B = len(lens)
    Wt = wl.layer_weights_v32(seed=43)
    act = wl.layer_activations(B, seed=43)
    cache, start = wl.decode_cache(np.asarray(lens), seed=43)
    cache_d = to_dev(cache)
    Wd = weights_to_dev(Wt)
    print(f"v32 decode fp8: lens={lens}", flush=True)
    qs, ws_ = [], []
    for b, L in enumerate(lens):
        q1, k1, w1 = dsa.v32_project(to_dev(act["x"][b:b + 1]), to_dev(act["c_q"][b:b + 1]), Wd, pos0=L - 1)
        cache_d[start[b] + L - 1] = k1[0]
        qs.append(q1)
        ws_.append(w1)
    q, w = torch.cat(qs), torch.cat(ws_)
    k8, ks = dsa.quantize_keys(cache_d)
    idx, sc = dsa.decode_fp8(q, w, k8, ks, torch.from_numpy(start).cuda(),
                             torch.from_numpy(np.asarray(lens, np.int32)).cuda(), max(lens), topk=2048)
    torch.cuda.synchronize()
    ke = np.round(np.log2(ks.cpu().numpy())).astype(np.int32)
    ref = oracle.rows_fp8(to_host(q).reshape(B, V32_H, D), to_host(w), k8.cpu().numpy(), ke, start,
                          np.asarray(lens) - 1, topk=2048, full=True)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    for b, L in enumerate(lens):
        check_row(L - 1, idx[b], sc[b], ref, b, 2048)
