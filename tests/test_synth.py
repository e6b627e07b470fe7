"""The seeded generator: determinism, independence of streams, distribution."""
import numpy as np

import synth
from synth import workloads as wl


def _f(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_deterministic_and_stream_independent():
    a = synth.normal_bf16((1000,), 0.0, 1.0, synth.Q, 0, 0)
    b = synth.normal_bf16((1000,), 0.0, 1.0, synth.Q, 0, 0)
    c = synth.normal_bf16((1000,), 0.0, 1.0, synth.K, 0, 0)
    d = synth.normal_bf16((1000,), 0.0, 1.0, synth.Q, 1, 0)
    e = synth.normal_bf16((1000,), 0.0, 1.0, synth.Q, 0, 1)
    assert np.array_equal(a, b)
    for other in (c, d, e):
        assert np.mean(a == other) < 0.05


def test_prefix_property():
    # counter-based: the first n elements do not depend on how many are drawn
    a = synth.normal_bf16((999,), 0.0, 1.0, synth.X)
    b = synth.normal_bf16((4000,), 0.0, 1.0, synth.X)
    assert np.array_equal(a, b[:999])


def test_range_is_a_slice_of_the_stream():
    full = synth.normal_bf16((5001,), 0.0, 1.0, synth.Q, 2, 3)
    for first, n in [(0, 10), (1, 10), (2, 7), (999, 1002), (4990, 11), (5000, 1)]:
        part = synth.normal_bf16((n,), 0.0, 1.0, synth.Q, 2, 3, first=first)
        assert np.array_equal(part, full[first:first + n])
    c = wl.chunk_inputs(300, 77, seed=4)
    s = wl.score_inputs(400, seed=4)
    assert np.array_equal(c["q"], s["q"][300:377])
    assert np.array_equal(c["w"], s["w"][300:377])
    assert np.array_equal(c["k"], s["k"][:377])


def test_moments_variance_convention():
    n = 400_000
    z = _f(synth.normal_bf16((n,), 0.0, 0.1, synth.W))
    assert abs(z.mean()) < 0.003
    assert abs(z.var() - 0.1) < 0.003          # 0.1 is the variance, std 0.316
    g = _f(synth.normal_bf16((n,), 1.0, 0.02, synth.GAMMA))
    assert abs(g.mean() - 1.0) < 0.002
    assert abs(g.var() - 0.02) < 0.001


def test_lengths():
    L = wl.decode_lengths(64)
    assert L.min() >= 32768 and L.max() <= 131072
    V = wl.varlen_lengths(16)
    assert V.min() >= 2048 and V.max() <= 32768
    assert np.array_equal(V, wl.varlen_lengths(16))
    cu = wl.cu_seqlens(V)
    assert cu[0] == 0 and cu[-1] == V.sum()
