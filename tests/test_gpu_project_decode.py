"""GPU parity of the projection GEMMs (with the key LayerNorm) and of decode."""
import numpy as np
import pytest
import torch

import oracle
from synth import workloads as wl
from tests.helpers import (check_projection, check_row, key_exact, linear_exact, to_dev, to_host,
                           weights_to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_token_idx_amd as m
    assert torch.cuda.is_available()
    return m


@pytest.mark.parametrize("T", [1, 37, 300])
def test_project_matches_oracle(dsa, T):
    Wt = wl.layer_weights(layer=1, seed=T)
    act = wl.layer_activations(T, seed=T)
    q, k, w = dsa.project(to_dev(act["x"]), to_dev(act["c_q"]), weights_to_dev(Wt))
    torch.cuda.synchronize()
    # each element: the bf16 rounding of an fp32 value within the accumulation radius of the
    # exact fp64 product (k: of its exact LayerNorm)
    fq = check_projection(to_host(q).reshape(T, -1), *linear_exact(act["c_q"], Wt["W_q"]), "q")
    fw = check_projection(to_host(w), *linear_exact(act["x"], Wt["W_w"]), "w")
    fk = check_projection(to_host(k), *key_exact(act["x"], Wt), "k")
    print(f"T={T}: fraction not correctly rounded q {fq:.1e} k {fk:.1e} w {fw:.1e}", flush=True)
    assert max(fq, fk, fw) < 1e-2


def test_project_strided_and_slots(dsa):
    T = 130
    Wt = wl.layer_weights(layer=2, seed=5)
    act = wl.layer_activations(T, seed=5)
    xw = np.zeros((T, 7168 + 64), np.uint16)
    xw[:, :7168] = act["x"]
    cw = np.zeros((T, 1536 + 8), np.uint16)
    cw[:, :1536] = act["c_q"]
    xd, cd = to_dev(xw), to_dev(cw)
    slots = np.random.default_rng(0).permutation(400)[:T].astype(np.int64)
    cache = torch.zeros((400, 128), dtype=torch.bfloat16, device="cuda")
    q, kc, w = dsa.project(xd[:, :7168], cd[:, :1536], weights_to_dev(Wt), k_out=cache,
                           k_slot=torch.from_numpy(slots).cuda())
    q2, k2, w2 = dsa.project(to_dev(act["x"]), to_dev(act["c_q"]), weights_to_dev(Wt))
    torch.cuda.synchronize()
    assert torch.equal(q.view(torch.int16), q2.view(torch.int16))
    assert torch.equal(w.view(torch.int16), w2.view(torch.int16))
    assert np.array_equal(to_host(kc)[slots], to_host(k2))
    untouched = np.setdiff1d(np.arange(400), slots)
    assert np.all(to_host(kc)[untouched] == 0)


def _decode_case(dsa, lens, seed, topk=2048):
    B = len(lens)
    Wt = wl.layer_weights(layer=0, seed=seed)
    act = wl.layer_activations(B, seed=seed)
    cache, start = wl.decode_cache(lens, seed=seed)
    cache_d = to_dev(cache)
    slots = (start + np.asarray(lens) - 1).astype(np.int64)
    q, _, w = dsa.project(to_dev(act["x"]), to_dev(act["c_q"]), weights_to_dev(Wt), k_out=cache_d,
                          k_slot=torch.from_numpy(slots).cuda())
    idx, sc = dsa.decode(q, w, cache_d, torch.from_numpy(start).cuda(),
                         torch.from_numpy(np.asarray(lens, np.int32)).cuda(), max(lens), topk=topk)
    torch.cuda.synchronize()
    return dict(q=to_host(q), w=to_host(w), cache=to_host(cache_d), start=start, idx=idx.cpu().numpy(),
                sc=sc.cpu().numpy(), Wt=Wt, act=act)


def test_decode_small(dsa):
    lens = [1, 2, 100, 2048, 2049, 5000, 4097]
    r = _decode_case(dsa, lens, seed=3)
    # stage-wise: oracle scores from the GPU's own q, w and cache
    ref = oracle.rows(r["q"], r["w"], r["cache"], r["start"], np.asarray(lens) - 1, topk=2048,
                      full=True)
    for b, L in enumerate(lens):
        check_row(L - 1, r["idx"][b], r["sc"][b], ref, b, 2048)
    # the new token's key in the cache: the rounding of a value within the accumulation
    # radius of the exact projection
    check_projection(r["cache"][r["start"] + np.asarray(lens) - 1], *key_exact(r["act"]["x"], r["Wt"]),
                     "new keys")


def test_decode_equals_prefill_last_row(dsa):
    lens = [3000, 2500]
    r = _decode_case(dsa, lens, seed=11)
    for b, L in enumerate(lens):
        a = r["start"][b]
        k = r["cache"][a:a + L]
        # prefill of a sequence whose last query is the decode query
        qs = np.zeros((L, 32, 128), np.uint16)
        ws = np.zeros((L, 32), np.uint16)
        qs[-1], ws[-1] = r["q"][b], r["w"][b]
        pi, ps = dsa.score_topk(to_dev(qs), to_dev(k), to_dev(ws), topk=2048)
        torch.cuda.synchronize()
        ref = oracle.rows(r["q"][[b]], r["w"][[b]], r["cache"], [a], [L - 1], topk=2048, full=True)
        check_row(L - 1, pi.cpu().numpy()[-1], ps.cpu().numpy()[-1], ref, 0, 2048)
        check_row(L - 1, r["idx"][b], r["sc"][b], ref, 0, 2048)


@pytest.mark.parametrize("topk", [1, 5, 100])
def test_decode_small_topk(dsa, topk):
    lens = [1, 50, 3000]
    r = _decode_case(dsa, lens, seed=topk, topk=topk)
    ref = oracle.rows(r["q"], r["w"], r["cache"], r["start"], np.asarray(lens) - 1, topk=topk,
                      full=True)
    for b, L in enumerate(lens):
        check_row(L - 1, r["idx"][b], r["sc"][b], ref, b, topk)


@pytest.mark.parametrize("topk", [2048, 64])
def test_decode_long_rows(dsa, topk):
    # caches longer than one register-held chunk of the decode select (16,384 scores) take its
    # sampled-threshold path; the longest length is not a multiple of 64 (padded row stride)
    lens = [16385, 20001, 33333]
    r = _decode_case(dsa, lens, seed=40 + topk, topk=topk)
    ref = oracle.rows(r["q"], r["w"], r["cache"], r["start"], np.asarray(lens) - 1, topk=topk,
                      full=True)
    for b, L in enumerate(lens):
        check_row(L - 1, r["idx"][b], r["sc"][b], ref, b, topk)
