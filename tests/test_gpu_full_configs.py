"""GPU parity at the full workload sizes, on outputs the oracle can compute one by one.

* one indexer layer at T = 8,192 and at T = 65,536 (project + score_topk, the launch the
  benchmark times): projections checked on sampled tokens against the fp32 summation
  bound; sampled rows checked end to end (oracle projections, scores and sort) and
  stage-wise (oracle scores and sort on the GPU's own q, k, w);
* decode with 64 sequences of U[32768, 131072] cached keys: sampled sequences;
* ragged prefill through 24 independent layers, 16 sequences of log-uniform length in
  [2048, 32768]: every layer stage-wise on sampled rows, projections on sampled tokens, and
  two layers end to end on the shortest sequence.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import workloads as wl
from tests.helpers import (U32, assert_bf16_within, check_row, check_row_e2e, projection_bounds,
                           to_dev, to_host, weights_to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_token_idx_amd as m
    assert torch.cuda.is_available()
    return m


def _check_projection_rows(q, k, w, act, Wt, rows):
    """GPU q, k, w rows against the exact products (fp32 summation bound + one ulp)."""
    eq, bq = projection_bounds(act["c_q"][rows], Wt["W_q"])
    ew, bw = projection_bounds(act["x"][rows], Wt["W_w"])
    ea, ba = projection_bounds(act["x"][rows], Wt["W_k"])
    ek = oracle.layernorm_f64(ea, Wt["gamma"], Wt["beta"], Wt["eps"])
    sigma = np.sqrt(ea.var(axis=1, keepdims=True) + Wt["eps"])
    gam = np.abs(oracle.bf16_to_f64(Wt["gamma"]))[None, :]
    bk = 2 * ba.max(axis=1, keepdims=True) / sigma * gam + 16 * U32 * (np.abs(ek) + 1)
    assert_bf16_within(q[rows].reshape(len(rows), -1), eq, bq, "q")
    assert_bf16_within(w[rows], ew, bw, "w")
    assert_bf16_within(k[rows], ek, bk, "k")


def _full_layer(dsa, T, n_rows, seed):
    Wt = wl.layer_weights(layer=0, seed=seed)
    act = wl.layer_activations(T, seed=seed)
    x, cq = to_dev(act["x"]), to_dev(act["c_q"])
    print(f"layer T={T}: project + score_topk on the GPU", flush=True)
    q, k, w = dsa.project(x, cq, weights_to_dev(Wt))
    idx, sc = dsa.score_topk(q, k, w, topk=2048)
    torch.cuda.synchronize()
    del x, cq
    gq, gk, gw = to_host(q), to_host(k), to_host(w)
    gi, gs = idx.cpu().numpy(), sc.cpu().numpy()
    rng = np.random.default_rng(T)
    rows = np.unique(np.concatenate([[0, 1, 2046, 2047, 2048, 2049, T // 2, T - 1],
                                     rng.integers(0, T, n_rows)]))
    rows = rows[rows < T]
    _check_projection_rows(gq, gk, gw, act, Wt, rows)
    # stage-wise: oracle scores + sort on the GPU's own q, k, w
    ref = oracle.prefill_rows(gq, gk, gw, rows, topk=2048, full=True)
    for r, t in enumerate(rows):
        check_row(t, gi[t], gs[t], ref, r, 2048)
    # end to end: the oracle's own projections (keys of the whole prefix of the last row)
    kmax = int(rows.max()) + 1
    print(f"layer T={T}: oracle keys for {kmax} tokens", flush=True)
    _, ok, _ = oracle.project(act["x"][:kmax], None, Wt, want=("k",))
    oq, _, ow = oracle.project(act["x"][rows], act["c_q"][rows], Wt, want=("q", "w"))
    ref2 = oracle.rows(oq, ow, ok, np.zeros(len(rows), np.int64), rows, topk=2048, full=True)
    for r, t in enumerate(rows):
        check_row_e2e(t, gi[t], gs[t], ref2, r, ref, r, 2048)


def test_full_layer_T8192(dsa):
    _full_layer(dsa, 8192, 56, seed=0)


def test_full_layer_T65536(dsa):
    _full_layer(dsa, 65536, 24, seed=0)


def test_decode_64_sequences(dsa):
    B = 64
    lens = wl.decode_lengths(B, seed=0)
    Wt = wl.layer_weights(layer=0, seed=1)
    act = wl.layer_activations(B, seed=1)
    cache, start = wl.decode_cache(lens, seed=0)
    cache_d = to_dev(cache)
    slots = (start + lens - 1).astype(np.int64)
    print(f"decode: B={B}, {int(lens.sum())} cached keys", flush=True)
    q, _, w = dsa.project(to_dev(act["x"]), to_dev(act["c_q"]), weights_to_dev(Wt), k_out=cache_d,
                          k_slot=torch.from_numpy(slots).cuda())
    idx, sc = dsa.decode(q, w, cache_d, torch.from_numpy(start).cuda(),
                         torch.from_numpy(lens.astype(np.int32)).cuda(), int(lens.max()), topk=2048)
    torch.cuda.synchronize()
    gq, gw = to_host(q), to_host(w)
    gi, gs = idx.cpu().numpy(), sc.cpu().numpy()
    new_keys = to_host(cache_d[torch.from_numpy(slots).cuda()])
    del cache_d
    sample = np.array([0, 1, int(np.argmax(lens)), int(np.argmin(lens)), 31, 63])
    cache[slots[sample]] = new_keys[sample]
    # stage-wise on the GPU's q, w and the cache (with the GPU's new keys)
    ref = oracle.rows(gq[sample], gw[sample], cache, start[sample], lens[sample] - 1, topk=2048,
                      full=True)
    for r, b in enumerate(sample):
        check_row(int(lens[b]) - 1, gi[b], gs[b], ref, r, 2048)
    # end to end: oracle projections of the new tokens
    oq, ok, ow = oracle.project(act["x"][sample], act["c_q"][sample], Wt)
    cache[slots[sample]] = ok
    ref2 = oracle.rows(oq, ow, cache, start[sample], lens[sample] - 1, topk=2048, full=True)
    for r, b in enumerate(sample):
        check_row_e2e(int(lens[b]) - 1, gi[b], gs[b], ref2, r, ref, r, 2048)


def test_varlen_24_layers(dsa):
    B, layers = 16, 24
    lens = wl.varlen_lengths(B, seed=0)
    cu = wl.cu_seqlens(lens)
    total = int(cu[-1])
    act = wl.layer_activations(total, seed=0)
    x, cq = to_dev(act["x"]), to_dev(act["c_q"])
    cu_d = torch.from_numpy(cu).cuda()
    shortest = int(np.argmin(lens))
    rng = np.random.default_rng(5)
    for layer in range(layers):
        Wt = wl.layer_weights(layer=layer, seed=0)
        print(f"varlen layer {layer}: {B} sequences, {total} tokens", flush=True)
        q, k, w = dsa.project(x, cq, weights_to_dev(Wt))
        idx, sc = dsa.score_topk_varlen(q, k, w, cu_d, int(lens.max()), topk=2048)
        torch.cuda.synchronize()

        def rows_of(t, r):
            return to_host(t[torch.from_numpy(np.asarray(r, np.int64)).cuda()])
        # projections on sampled tokens
        toks = np.unique(rng.integers(0, total, 16))
        _check_projection_rows(rows_of(q, toks), rows_of(k, toks), rows_of(w, toks),
                               {"x": act["x"][toks], "c_q": act["c_q"][toks]}, Wt,
                               np.arange(len(toks)))
        # stage-wise rows of two sequences
        for b in (shortest, int(rng.integers(0, B))):
            a0, L = int(cu[b]), int(lens[b])
            rows = np.unique(np.concatenate([[0, 2047, L - 1], rng.integers(0, L, 5)]))
            rows = rows[rows < L]
            gk = to_host(k[a0:a0 + L])
            gi = idx[a0 + rows].cpu().numpy()
            gs = sc[a0 + rows].cpu().numpy()
            ref = oracle.rows(rows_of(q, a0 + rows), rows_of(w, a0 + rows), gk,
                              np.zeros(len(rows), np.int64), rows, topk=2048, full=True)
            for r, t in enumerate(rows):
                check_row(int(t), gi[r], gs[r], ref, r, 2048)
        if layer in (0, layers - 1):
            # end to end on the shortest sequence: oracle projections of all its tokens
            a0, L = int(cu[shortest]), int(lens[shortest])
            oq, ok, ow = oracle.project(act["x"][a0:a0 + L], act["c_q"][a0:a0 + L], Wt)
            rows = np.array(sorted(set([0, 1, 2047, L // 2, L - 1]) & set(range(L))))
            gi = idx[a0 + rows].cpu().numpy()
            gs = sc[a0 + rows].cpu().numpy()
            ref2 = oracle.prefill_rows(oq, ok, ow, rows, topk=2048, full=True)
            ref_sw = oracle.rows(rows_of(q, a0 + rows), rows_of(w, a0 + rows), to_host(k[a0:a0 + L]),
                                 np.zeros(len(rows), np.int64), rows, topk=2048, full=True)
            for r, t in enumerate(rows):
                check_row_e2e(int(t), gi[r], gs[r], ref2, r, ref_sw, r, 2048)
