"""The paths of the prefill top-k, each forced by its input and checked against the oracle:

* rows of at most 4,096 keys keep every key; longer rows keep the keys at or above a
  threshold placed from one sampled key per 32-key stratum, and select exactly among them;
* a row whose sample overshoots (fewer kept keys than topk) and a row whose kept keys overflow
  their list (all scores equal) are both scored again in full and selected from all scores;
* sequences longer than one filter pass (65,536 rows) and than one sample buffer;
* one call over a 1,048,576-token sequence (no T x T storage), on sampled rows;
* a ring wait that runs out of polls is reported (status word, index -2) instead of giving
  wrong selections.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import workloads as wl
from tests.helpers import check_row, to_dev, to_host

pytestmark = pytest.mark.gpu

STRIDE = 32          # keys per sample stratum
ALL_KEYS = 4096      # rows of at most this many keys keep every key


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_token_idx_amd as m
    assert torch.cuda.is_available()
    return m


def _mix32(x):
    """The lowbias32 integer mixer (C. Wellons), on uint32 numpy arrays."""
    x = x.astype(np.uint64) & 0xFFFFFFFF
    x ^= x >> 16
    x = (x * 0x7FEB352D) & 0xFFFFFFFF
    x ^= x >> 15
    x = (x * 0x846CA68B) & 0xFFFFFFFF
    x ^= x >> 16
    return x


def sampled_positions(n):
    """Key positions the library samples in a sequence of n keys: one per full stratum."""
    j = np.arange(n // STRIDE, dtype=np.uint64)
    return (j * STRIDE + (_mix32(j + 0x9E3779B9) & (STRIDE - 1))).astype(np.int64)


def _run(dsa, q, k, w, topk):
    idx, sc = dsa.score_topk(to_dev(q), to_dev(k), to_dev(w), topk=topk)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy()


def _bf(x):
    return oracle.f64_to_bf16(np.asarray(x, np.float64))


def test_sample_overshoot_falls_back(dsa):
    """Every sampled key scores far above the rest, so a row's threshold (the r-th largest
    sample, r about 118) keeps about r keys: fewer than topk.  The row is scored again in full
    and selected exactly: all its sampled keys plus the best of the others."""
    T, topk = 9000, 2048
    rng = np.random.default_rng(41)
    q = _bf(np.abs(rng.standard_normal((T, 32, 128))))
    w = _bf(rng.uniform(0.5, 1.0, (T, 32)))
    kf = rng.standard_normal((T, 128))
    kf[sampled_positions(T)] = 4.0
    k = _bf(kf)
    print("overshoot: T=9000 with planted sampled keys", flush=True)
    gi, gs = _run(dsa, q, k, w, topk)
    rows = [100, 4095, 4096, 4097, 6000, 7777, 8999]
    ref = oracle.prefill_rows(q, k, w, rows, topk=topk, full=True)
    for r, t in enumerate(rows):
        check_row(t, gi[t], gs[t], ref, r, topk)
        planted = set(sampled_positions(t + 1).tolist())
        assert planted <= set(gi[t][gi[t] >= 0].tolist())


def test_all_equal_scores_overflow_falls_back(dsa):
    """Every key of a row scores the same, so every key reaches the threshold: rows of more than
    6,144 keys overflow their list and are selected from their full rescoring, rows below are
    selected from their lists; either way the lowest topk indices win the tie."""
    T = 9000
    rng = np.random.default_rng(43)
    q = _bf(rng.standard_normal((T, 32, 128)))
    w = _bf(rng.standard_normal((T, 32)))
    k = np.repeat(_bf(rng.standard_normal((1, 128))), T, axis=0)
    print("all-equal: T=9000", flush=True)
    for topk in (2048, 100):
        gi, gs = _run(dsa, q, k, w, topk)
        for t in (5000, 6143, 6144, 6145, 8999):
            assert np.array_equal(gi[t], np.arange(topk)), t
            assert np.all(gs[t] == gs[t][0])
        rows = [6200, 8999]
        ref = oracle.prefill_rows(q, k, w, rows, topk=topk, full=True)
        for r, t in enumerate(rows):
            check_row(t, gi[t], gs[t], ref, r, topk)


def test_sequence_longer_than_one_filter_pass(dsa):
    """70,000 rows: two filter passes (65,536 rows each at most) and two sample sub-chunks."""
    T = 70000
    s = wl.score_inputs(T, seed=47)
    print("two filter passes: T=70000", flush=True)
    gi, gs = _run(dsa, s["q"], s["k"], s["w"], 2048)
    rows = [0, 4095, 4096, 58239, 58240, 65535, 65536, 65537, 69999]
    ref = oracle.prefill_rows(s["q"], s["k"], s["w"], rows, topk=2048, full=True)
    for r, t in enumerate(rows):
        check_row(t, gi[t], gs[t], ref, r, 2048)


def test_one_call_over_a_million_tokens(dsa):
    """A single dsa_idx_score_topk call at T = 1,048,576: its workspace is a few GB (the score
    triangle would be 2.2 TB).  Inputs come from torch's seeded generator on the device with
    the workload's distributions; sampled rows are checked against the oracle."""
    T = 1 << 20
    ws_bytes = dsa.workspace_size(dsa.OP_SCORE_TOPK, T, topk=2048)
    assert ws_bytes < 6 * 2 ** 30
    g = torch.Generator(device="cuda")
    g.manual_seed(53)
    print(f"T=2^20: inputs on the device, workspace {ws_bytes / 2 ** 30:.2f} GiB", flush=True)
    q = torch.randn((T, 32, 128), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((T, 128), generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn((T, 32), generator=g, device="cuda") * 0.1 ** 0.5).to(torch.bfloat16)
    print("T=2^20: score_topk", flush=True)
    idx, sc = dsa.score_topk(q, k, w, topk=2048)
    torch.cuda.synchronize()
    rows = np.array([0, 2047, 2048, 65535, 65536, 300001, 777777, T - 1])
    sel = torch.from_numpy(rows).cuda()
    gi, gs = idx[sel].cpu().numpy(), sc[sel].cpu().numpy()
    qh, wh, kh = to_host(q[sel]), to_host(w[sel]), to_host(k)
    del q, w, idx, sc
    print("T=2^20: oracle rows", flush=True)
    ref = oracle.rows(qh, wh, kh, np.zeros(len(rows), np.int64), rows, topk=2048, full=True)
    for r, t in enumerate(rows):
        check_row(int(t), gi[r], gs[r], ref, r, 2048)


def test_stalled_ring_wait_is_reported(dsa):
    """With no polls allowed, a score kernel's ring waits give up: the call must still end,
    mark its outputs invalid (index -2) and report ESTALL through the workspace status."""
    T = 3000
    s = wl.score_inputs(T, seed=59)
    q, k, w = to_dev(s["q"]), to_dev(s["k"]), to_dev(s["w"])
    ws = torch.empty(dsa.workspace_size(dsa.OP_SCORE_TOPK, T, topk=64), dtype=torch.uint8, device="cuda")
    prev = dsa.set_wait_budget(0)
    try:
        print("stall: score_topk with a zero wait budget", flush=True)
        idx, sc = dsa.score_topk(q, k, w, topk=64, ws=ws)
        with pytest.raises(dsa.DsaIdxError) as e:
            dsa.workspace_status(ws)
        assert e.value.code == dsa.ESTALL
        assert (idx == -2).all() and torch.isnan(sc).all()
        rws = dsa.prefill_rows_workspace(T)
        dsa.prefill_scores(q, k, w, rws)
        ridx, _ = dsa.prefill_select(T, rws, topk=64)
        with pytest.raises(dsa.DsaIdxError):
            dsa.workspace_status(rws)
        assert (ridx == -2).all()
    finally:
        dsa.set_wait_budget(prev)
    print("stall: default budget again", flush=True)
    idx, sc = dsa.score_topk(q, k, w, topk=64, ws=ws)
    dsa.workspace_status(ws)
    gi, gs = idx.cpu().numpy(), sc.cpu().numpy()
    rows = [0, 63, 64, 2999]
    ref = oracle.prefill_rows(s["q"], s["k"], s["w"], rows, topk=64, full=True)
    for r, t in enumerate(rows):
        check_row(t, gi[t], gs[t], ref, r, 64)
