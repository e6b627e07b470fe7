"""Pins of the CPU oracle to facts fixed outside itself (CPU only).

Each test ties a part of the oracle to the pages' figures, to exact
mathematics, to a library routine for a special case, or to brute force, so
that a dropped term, a wrong sign or index, or a transposed operand fails here.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import D, H, HIDDEN, QLAT, QOUT, TOPK
import synth
from synth import workloads as wl


def bf(x):
    """Exactly representable values -> bf16 patterns (via float32 truncation, exact here)."""
    a = np.asarray(x, dtype=np.float32)
    bits = a.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


# ----------------------------------------------------------------- parameter count
def test_param_count_matches_pages():
    # Sparse-attention row: "7.44M BF16 parameters per layer"; low-precision row of the
    # "Kimi K3.1 Pro vs GLM-5" page: the new indexer has 178.5M parameters over 24 layers.
    n = oracle.param_count()
    assert n == 1536 * 4096 + 7168 * 128 + 7168 * 32 + 2 * 128 == 7_438_592
    assert f"{n / 1e6:.2f}" == "7.44"
    assert f"{24 * n / 1e6:.1f}" == "178.5"
    # Projection biases would add 4,096 + 128 + 32 per layer and print as 178.6M: ruled out.
    assert f"{24 * (n + 4096 + 128 + 32) / 1e6:.1f}" == "178.6"
    d = oracle.dims()
    assert (d["heads"], d["dim"], d["qlat"], d["qout"], d["hidden"], d["topk"]) == \
        (32, 128, 1536, 4096, 7168, 2048)
    assert d["heads"] * d["dim"] == d["qout"]


# ----------------------------------------------------------------- bf16 rounding
RNE_CASES = [
    # (value, expected bf16 bits) -- derived from the bf16 format: 1 sign, 8 exponent,
    # 7 stored mantissa bits; ulp at 1.0 is 2^-7.
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),                   # tie between 1 and 1+2^-7 -> even (1)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),               # tie between 1+2^-7 (odd) and 1+2^-6 -> even
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),      # just above the tie: up (fp32 detour gives 0x3F80)
    (1.0 + 2.0 ** -8 - 2.0 ** -40, 0x3F80),      # just below the tie: down
    (-(1.0 + 3 * 2.0 ** -8), 0xBF82),
    (3.0, 0x4040),
    (-2.0, 0xC000),
    ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),      # largest finite
    ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),      # tie above the largest finite -> even -> inf
    (1e300, 0x7F80),
    (-1e300, 0xFF80),
    (2.0 ** -126, 0x0080),                       # smallest normal
    (2.0 ** -133, 0x0001),                       # smallest subnormal
    (2.0 ** -134, 0x0000),                       # tie between 0 and 2^-133 -> even (0)
    (1.5 * 2.0 ** -134, 0x0001),
    (3 * 2.0 ** -134, 0x0002),                   # tie between 2^-133 (odd) and 2^-132 -> even
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (math.inf, 0x7F80),
    (-math.inf, 0xFF80),
]


@pytest.mark.parametrize("x,bits", RNE_CASES)
def test_rne_constructed(x, bits):
    assert int(oracle.f64_to_bf16(np.array([x]))[0]) == bits


def test_rne_nan_and_widen():
    assert int(oracle.f64_to_bf16(np.array([math.nan]))[0]) == 0x7FC0
    assert oracle.bf16_to_f64(np.array([0x3F80, 0xC000, 0x0001], np.uint16)).tolist() == \
        [1.0, -2.0, 2.0 ** -133]


def test_rne_is_nearest_on_random_values():
    # For random doubles the result must be a nearest bf16 neighbour (brute force over the
    # two candidates bracketing x).
    rng = np.random.default_rng(1)
    x = rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))
    b = oracle.f64_to_bf16(x)
    v = oracle.bf16_to_f64(b)
    up = oracle.bf16_to_f64((b.astype(np.int64) + 1).astype(np.uint16))
    dn = oracle.bf16_to_f64((b.astype(np.int64) - 1).astype(np.uint16))
    assert np.all(np.abs(v - x) <= np.abs(up - x))
    assert np.all(np.abs(v - x) <= np.abs(dn - x))


# ----------------------------------------------------------------- projections
@pytest.fixture(scope="module")
def small_layer():
    Wt = wl.layer_weights(layer=3)
    act = wl.layer_activations(24, layer=3)
    return Wt, act


def test_linear_matches_numpy_matmul(small_layer):
    Wt, act = small_layer
    for A, W in ((act["c_q"], Wt["W_q"]), (act["x"], Wt["W_k"]), (act["x"], Wt["W_w"])):
        ref = oracle.bf16_to_f64(A) @ oracle.bf16_to_f64(W)
        got = oracle.linear_f64(A, W)
        scale = np.abs(ref).max()
        assert np.max(np.abs(got - ref)) <= 1e-12 * scale


def test_project_is_rounded_linear_and_layernorm(small_layer):
    Wt, act = small_layer
    q, k, w = oracle.project(act["x"], act["c_q"], Wt)
    qf = oracle.bf16_to_f64(act["c_q"]) @ oracle.bf16_to_f64(Wt["W_q"])
    wf = oracle.bf16_to_f64(act["x"]) @ oracle.bf16_to_f64(Wt["W_w"])
    a = oracle.bf16_to_f64(act["x"]) @ oracle.bf16_to_f64(Wt["W_k"])
    kf = torch.nn.functional.layer_norm(
        torch.from_numpy(a), (D,), weight=torch.from_numpy(oracle.bf16_to_f64(Wt["gamma"])),
        bias=torch.from_numpy(oracle.bf16_to_f64(Wt["beta"])), eps=Wt["eps"]).numpy()
    # post-rounding agreement; a disagreement is only allowed where the reference value
    # sits within 1e-12 (relative) of a rounding midpoint
    for got, ref in ((q.reshape(len(q), -1), qf), (k, kf), (w, wf)):
        want = oracle.f64_to_bf16(ref)
        diff = got != want
        if diff.any():
            near = oracle.f64_to_bf16(ref * (1 + 1e-12)) != oracle.f64_to_bf16(ref * (1 - 1e-12))
            assert np.all(near[diff])
        assert diff.mean() < 1e-3


def test_layernorm_matches_torch_and_invariants():
    rng = np.random.default_rng(7)
    a = rng.standard_normal((8, D)) * 3 + 1
    g = np.full(D, 0x3F80, np.uint16)
    b0 = np.zeros(D, np.uint16)
    gam = synth.normal_bf16((D,), 1.0, 0.02, synth.GAMMA)
    bet = synth.normal_bf16((D,), 0.0, 0.02, synth.BETA)
    eps = 1e-6
    got = oracle.layernorm_f64(a, gam, bet, eps)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(a), (D,),
                                         torch.from_numpy(oracle.bf16_to_f64(gam)),
                                         torch.from_numpy(oracle.bf16_to_f64(bet)), eps).numpy()
    assert np.max(np.abs(got - ref)) < 1e-12
    # shift invariance
    assert np.max(np.abs(oracle.layernorm_f64(a + 1024.0, gam, bet, eps) - got)) < 1e-9
    # scale invariance up to the eps term
    assert np.max(np.abs(oracle.layernorm_f64(a * 4.0, gam, bet, eps) - got)) < 1e-5
    # gamma = 1, beta = 0: zero mean, mean square var/(var + eps)
    n = oracle.layernorm_f64(a, g, b0, eps)
    var = a.var(axis=1)
    assert np.max(np.abs(n.mean(axis=1))) < 1e-12
    assert np.max(np.abs((n ** 2).mean(axis=1) - var / (var + eps))) < 1e-12


def test_layernorm_is_not_rmsnorm():
    # a mean-shifted key changes an RMS-normalised output but not the LayerNorm output
    a = np.linspace(-1, 3, D)[None, :]
    g = np.full(D, 0x3F80, np.uint16)
    b0 = np.zeros(D, np.uint16)
    out = oracle.layernorm_f64(a, g, b0, 1e-6)
    assert abs(out.mean()) < 1e-12
    rms = a / np.sqrt((a ** 2).mean() + 1e-6)
    assert np.max(np.abs(out - rms)) > 0.1


# ----------------------------------------------------------------- scores: hand example
def _hand_inputs(gh, pad=False):
    q = np.array(gh["q"], np.float32)
    k = np.array(gh["k"], np.float32)
    w = np.array(gh["w"], np.float32)
    if pad:
        qp = np.zeros((q.shape[0], H, D), np.float32)
        qp[:, :q.shape[1], :q.shape[2]] = q
        kp = np.zeros((k.shape[0], D), np.float32)
        kp[:, :k.shape[1]] = k
        wp = np.zeros((w.shape[0], H), np.float32)
        wp[:, :w.shape[1]] = w
        q, k, w = qp, kp, wp
    return bf(q), bf(k), bf(w)


@pytest.mark.parametrize("pad", [False, True])
def test_hand_example(golden_hand, pad):
    gh = golden_hand
    q, k, w = _hand_inputs(gh, pad)
    for t in range(gh["T"]):
        I = oracle.scores(q[t], w[t], k, t + 1)
        assert I.tolist() == gh["expected_scores"][t]
    for name, kk in (("topk2", 2), ("topk1", 1)):
        out = oracle.prefill_rows(q, k, w, [0, 1, 2], topk=kk)
        for t in range(3):
            sel = [int(i) for i in out["idx"][t] if i >= 0]
            assert sel == gh["expected_selection"][name][t]
    nv = gh["negative_w_variant"]
    w2 = w.copy()
    w2[nv["row"], :2] = bf(np.array(nv["w"], np.float32))
    assert oracle.scores(q[2], w2[2], k, 3).tolist() == nv["expected_scores"]
    for name, kk in (("topk2", 2), ("topk1", 1)):
        idx, _, _, _ = oracle.topk(np.array(nv["expected_scores"]), kk)
        assert [int(i) for i in idx if i >= 0] == nv["expected_selection"][name]


def test_hand_example_catches_folded_heads(golden_hand):
    # A planted mistake in a copy of the oracle's formula -- sum_h w_h q_h folded before the
    # dot, no ReLU -- must disagree with the fixture on row 2.
    gh = golden_hand
    q = np.array(gh["q"], np.float64)
    k = np.array(gh["k"], np.float64)
    w = np.array(gh["w"], np.float64)
    folded = (w[2][:, None] * q[2]).sum(0) @ k.T
    assert folded.tolist() == gh["folded_no_relu_row2_scores"]
    assert folded.tolist() != gh["expected_scores"][2]


# ----------------------------------------------------------------- scores: special cases
def test_single_head_nonnegative_is_causal_gemm():
    rng = np.random.default_rng(3)
    T = 50
    qv = np.abs(rng.standard_normal((T, D))).astype(np.float32)
    kv = np.abs(rng.standard_normal((T, D))).astype(np.float32)
    q = np.zeros((T, H, D), np.uint16)
    q[:, 0] = oracle.f64_to_bf16(qv)
    k = oracle.f64_to_bf16(kv)
    w = np.zeros((T, H), np.uint16)
    w[:, 0] = 0x3F80
    G = oracle.bf16_to_f64(q[:, 0]) @ oracle.bf16_to_f64(k).T   # exact: bf16 products, few bits
    for t in (0, 1, 17, T - 1):
        assert np.array_equal(oracle.scores(q[t], w[t], k, t + 1), G[t, :t + 1])


@pytest.fixture(scope="module")
def small_scores():
    return wl.score_inputs(300, seed=5)


def test_power_of_two_invariances(small_scores):
    s = small_scores
    q, k, w = s["q"], s["k"], s["w"]
    rows = [0, 5, 150, 299]
    base = oracle.prefill_rows(q, k, w, rows, topk=64, full=True)
    sc2 = lambda b, j: oracle.f64_to_bf16(oracle.bf16_to_f64(b) * 2.0 ** j)
    # (i) w * 2^j -> I * 2^j, same selection
    o1 = oracle.prefill_rows(q, k, sc2(w, 3), rows, topk=64, full=True)
    # (ii) k * 2^j -> I * 2^j
    o2 = oracle.prefill_rows(q, sc2(k, -2), w, rows, topk=64, full=True)
    # (iii) (q_h * 2^j, w_h * 2^-j) -> I unchanged
    q3, w3 = q.copy(), w.copy()
    q3[:, 7] = sc2(q[:, 7], 4)
    w3[:, 7] = sc2(w[:, 7], -4)
    o3 = oracle.prefill_rows(q3, k, w3, rows, topk=64, full=True)
    for r in range(len(rows)):
        assert np.array_equal(o1["full"][r], base["full"][r] * 8)
        assert np.array_equal(o2["full"][r], base["full"][r] / 4)
        assert np.array_equal(o3["full"][r], base["full"][r])
        for o in (o1, o2, o3):
            assert np.array_equal(o["idx"][r], base["idx"][r])


def test_head_permutation(small_scores):
    s = small_scores
    perm = np.random.default_rng(0).permutation(H)
    rows = [10, 299]
    a = oracle.prefill_rows(s["q"], s["k"], s["w"], rows, topk=64, full=True)
    b = oracle.prefill_rows(s["q"][:, perm], s["k"], s["w"][:, perm], rows, topk=64, full=True)
    for r in range(len(rows)):
        tol = 1e-12 * a["maxabs"][r]
        assert np.max(np.abs(a["full"][r] - b["full"][r])) <= tol
        diff = set(a["idx"][r].tolist()) ^ set(b["idx"][r].tolist())
        assert all(abs(a["full"][r][i] - a["tau"][r]) <= tol for i in diff if i >= 0)


def test_relu_matters(small_scores):
    # dropping the ReLU (planted in a numpy copy of the formula) changes the scores
    s = small_scores
    t = 200
    I = oracle.scores(s["q"][t], s["w"][t], s["k"], t + 1)
    qd = oracle.bf16_to_f64(s["q"][t])
    kd = oracle.bf16_to_f64(s["k"][:t + 1])
    wd = oracle.bf16_to_f64(s["w"][t])
    with_relu = (wd[:, None] * np.maximum(qd @ kd.T, 0)).sum(0)
    no_relu = (wd[:, None] * (qd @ kd.T)).sum(0)
    assert np.max(np.abs(I - with_relu)) <= 1e-12 * np.abs(I).max()
    assert np.max(np.abs(I - no_relu)) > 1.0


def test_causality(small_scores):
    s = small_scores
    k2 = s["k"].copy()
    k2[101:] = synth.normal_bf16(k2[101:].shape, 0.0, 1.0, synth.K, 9)
    a = oracle.prefill_rows(s["q"], s["k"], s["w"], [100], topk=32, full=True)
    b = oracle.prefill_rows(s["q"], k2, s["w"], [100], topk=32, full=True)
    assert np.array_equal(a["full"][0], b["full"][0])
    assert np.array_equal(a["idx"], b["idx"])


# ----------------------------------------------------------------- selection
def _check_defining_property(I, sel, kk):
    n = len(I)
    assert len(sel) == min(kk, n) and len(set(sel)) == len(sel)
    assert all(0 <= s < n for s in sel)
    S = set(sel)
    for a in sel:
        for b in range(n):
            if b in S:
                continue
            assert I[a] > I[b] or (I[a] == I[b] and a < b)


@pytest.mark.parametrize("kk", [1, 2, 3, 8, 16])
def test_bruteforce_tiny_with_ties(kk):
    rng = np.random.default_rng(kk)
    Hh, Dd, T = 4, 8, 40
    # coarse values force many exact ties in the scores
    q = oracle.f64_to_bf16(rng.integers(-2, 3, (T, Hh, Dd)).astype(np.float64))
    k = oracle.f64_to_bf16(rng.integers(-2, 3, (T, Dd)).astype(np.float64))
    w = oracle.f64_to_bf16(rng.integers(-1, 3, (T, Hh)).astype(np.float64) * 0.5)
    out = oracle.prefill_rows(q, k, w, np.arange(T), topk=kk, full=True)
    saw_tie = False
    for t in range(T):
        I = out["full"][t]
        sel = [int(i) for i in out["idx"][t] if i >= 0]
        assert sel == sorted(sel)
        _check_defining_property(I, sel, kk)
        ref = sorted(np.argsort(-I, kind="stable")[:kk].tolist())
        assert sel == ref
        saw_tie |= len(np.unique(I)) < len(I)
        # the returned scores are the scores of the returned indices
        assert np.array_equal(out["score"][t][:len(sel)], I[sel])
        assert np.all(np.isneginf(out["score"][t][len(sel):]))
        assert np.all(out["idx"][t][len(sel):] == -1)
    assert saw_tie


def test_negative_zero_ties_positive_zero():
    I = np.array([0.0, -0.0, 0.0, -1.0])
    idx, _, tau, _ = oracle.topk(I, 2)
    assert idx.tolist() == [0, 1]
    idx, _, _, _ = oracle.topk(np.array([-0.0, 0.0]), 1)
    assert idx.tolist() == [0]


def test_short_rows_rule():
    # t < 2048 keeps every causal token; row 2047 keeps all 2,048; row 2048 drops one
    s = wl.score_inputs(2050, seed=11)
    rows = [0, 1, 2046, 2047, 2048, 2049]
    out = oracle.prefill_rows(s["q"], s["k"], s["w"], rows, topk=TOPK, full=True)
    for r, t in enumerate(rows):
        sel = out["idx"][r]
        if t <= 2047:
            assert sel[:t + 1].tolist() == list(range(t + 1))
            assert np.all(sel[t + 1:] == -1)
            assert out["tau"][r] == -math.inf
        else:
            kept = set(sel.tolist())
            assert len(kept) == TOPK and -1 not in kept
            dropped = sorted(set(range(t + 1)) - kept)
            assert len(dropped) == t + 1 - TOPK
            I = out["full"][r]
            assert max(I[dropped]) <= out["tau"][r]


def test_rows_offsets_equal_sliced_calls():
    # varlen/decode addressing: a row scored at an offset into a packed key array equals the
    # same row scored on its own slice
    s = wl.score_inputs(120, seed=2)
    off = 37
    a = oracle.rows(s["q"][[90]], s["w"][[90]], s["k"], [off], [50], topk=16, full=True)
    b = oracle.rows(s["q"][[90]], s["w"][[90]], s["k"][off:], [0], [50], topk=16, full=True)
    assert np.array_equal(a["full"][0], b["full"][0])
    assert np.array_equal(a["idx"], b["idx"])
