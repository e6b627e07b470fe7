"""Pins of the oracle's DeepSeek-V3.2-shaped indexer (64 heads, rotary step on 64 of the 128
dims), on the CPU.

The pages fix the head count (sparse-attention row of the "Qwen3.5-397B-A17B vs Kimi K3.1 Pro"
page) and that 64 of the 128 dims are rotated (RoPE row of the "Kimi K3.1 Pro vs Gemma 4 31B"
page).  The rest of the rotary step is a reading: adjacent pairs (2i, 2i+1) of dims 0..63,
angle pos * 10^4^(-2i/64).  The pins below hold for any rotary step of that kind, whatever its
frequencies, and break for the plausible slips: a sign, the wrong pair or dims, rotating q and
k differently, or a position that is not relative in the end; the head split pins the sum the
GPU path computes in two halves."""
import numpy as np

import oracle
from oracle import D, V32_H
from synth import workloads as wl


def _rng(seed):
    return np.random.default_rng(seed)


def test_position_zero_is_the_identity():
    v = _rng(0).standard_normal((3, 5, D))
    assert np.array_equal(oracle.rope_f64(v, np.zeros(3, np.int64)), v)


def test_upper_dims_are_not_rotated_and_lower_ones_are():
    v = _rng(1).standard_normal((4, D))
    r = oracle.rope_f64(v, np.array([1, 17, 1000, 999_999]))
    assert np.array_equal(r[:, 64:], v[:, 64:])
    assert np.all(np.abs(r[:, :64] - v[:, :64]).max(axis=1) > 1e-3)


def test_pairs_keep_their_length():
    v = _rng(2).standard_normal((6, 2, D))
    r = oracle.rope_f64(v, np.array([3, 50, 4096, 65535, 10 ** 6, 7]))
    n0 = v[..., 0:64:2] ** 2 + v[..., 1:64:2] ** 2
    n1 = r[..., 0:64:2] ** 2 + r[..., 1:64:2] ** 2
    assert np.allclose(n1, n0, rtol=1e-12, atol=0)


def test_dot_products_depend_on_the_offset_only():
    rng = _rng(3)
    q, k = rng.standard_normal((1, D)), rng.standard_normal((1, D))
    for m, n in [(5, 2), (1000, 0), (70_000, 65_000), (3, 9)]:
        d0 = float(oracle.rope_f64(q, [m])[0] @ oracle.rope_f64(k, [n])[0])
        for shift in (1, 123, 500_000):
            d1 = float(oracle.rope_f64(q, [m + shift])[0] @ oracle.rope_f64(k, [n + shift])[0])
            assert abs(d1 - d0) <= 1e-9 * (1 + abs(d0))
        # and equal to the query turned by the offset against the unturned key
        d2 = float(oracle.rope_f64(q, [m - n])[0] @ k[0])
        assert abs(d2 - d0) <= 1e-9 * (1 + abs(d0))


def test_rotations_compose():
    v = _rng(4).standard_normal((1, D))
    a = oracle.rope_f64(oracle.rope_f64(v, [300]), [4000])
    b = oracle.rope_f64(v, [4300])
    assert np.allclose(a, b, rtol=0, atol=1e-10)


def test_frequency_ladder():
    # at position 1, pair i turns its first unit vector by theta^(-2i/64): a ladder from 1 rad
    # down by the same ratio at each step, pair i staying in dims 2i and 2i + 1
    ang = []
    for i in range(32):
        e = np.zeros((1, D))
        e[0, 2 * i] = 1.0
        r = oracle.rope_f64(e, [1])[0]
        moved = np.flatnonzero(np.abs(r - e[0]) > 0)
        assert set(moved.tolist()) <= {2 * i, 2 * i + 1}
        ang.append(np.arctan2(r[2 * i + 1], r[2 * i]))
    ang = np.array(ang)
    assert abs(ang[0] - 1.0) < 1e-15
    ratio = ang[1:] / ang[:-1]
    assert np.allclose(ratio, 10000.0 ** (-2.0 / 64), rtol=1e-12)


def test_projection_matches_the_k31_projection_on_shared_columns():
    # with the first 4,096 query columns and 32 weight columns, the unrotated parts (position
    # 0) equal the K3.1 oracle's projections, computed by the separate C path
    Wt = wl.layer_weights_v32(seed=5)
    act = wl.layer_activations(3, seed=5)
    q, k, w = oracle.project_v32(act["x"][:1], act["c_q"][:1], Wt, pos0=0)
    W31 = dict(Wt)
    W31["W_q"] = np.ascontiguousarray(Wt["W_q"][:, :4096])
    W31["W_w"] = np.ascontiguousarray(Wt["W_w"][:, :32])
    q31, k31, w31 = oracle.project(act["x"][:1], act["c_q"][:1], W31)
    assert q.shape == (1, V32_H, D) and w.shape == (1, V32_H)
    assert np.array_equal(q[:, :32], q31) and np.array_equal(k, k31) and np.array_equal(w[:, :32], w31)
    # later positions rotate q and k (dims < 64 only), and leave w alone
    q2, k2, w2 = oracle.project_v32(act["x"], act["c_q"], Wt, pos0=9)
    q0, k0, _ = oracle.project_v32(act["x"], act["c_q"], Wt, pos0=0)
    assert np.array_equal(q2[..., 64:], q0[..., 64:]) and np.array_equal(k2[:, 64:], k0[:, 64:])
    assert not np.array_equal(q2[..., :64], q0[..., :64])
    assert np.array_equal(w2, oracle.project_v32(act["x"], act["c_q"], Wt, want=("w",))[2])


def test_scores_split_over_the_two_head_halves():
    rng = _rng(6)
    T = 40
    q = oracle.f64_to_bf16(rng.standard_normal((T, V32_H, D)))
    k = oracle.f64_to_bf16(rng.standard_normal((T, D)))
    w = oracle.f64_to_bf16(rng.standard_normal((T, V32_H)) * 0.3)
    for t in (0, 7, 39):
        full = oracle.scores(q[t], w[t], k, t + 1)
        lo = oracle.scores(q[t, :32], w[t, :32], k, t + 1)
        hi = oracle.scores(q[t, 32:], w[t, 32:], k, t + 1)
        assert np.allclose(full, lo + hi, rtol=1e-13, atol=1e-12)
