"""Pins of the oracle's FP8 (OCP E4M3) key-cache path, on the CPU.

The format reading: E4M3 codes (bias 7, 448 the largest finite value, no infinities) with one
power-of-two scale per vector, the smallest 2^e with max|x| <= 448 * 2^e, so the only rounding
is round-to-nearest-even onto E4M3 ("Kimi K3.1 Pro vs GLM-5" compare page, low-precision row:
serving engines cache the indexer keys in FP8; the pages give no format or scale)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import D, H


def _torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _torch_encode_f32(x32):
    """torch's float32 -> float8_e4m3fn conversion (a single rounding from float32)."""
    t = torch.from_numpy(np.asarray(x32, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_to_f64(codes)
    ref = _torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert nan.sum() == 2 and set(codes[nan].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(mine[~nan], ref[~nan])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6


def test_encode_inverts_decode():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.e4m3_to_f64(codes)
    assert np.array_equal(oracle.f64_to_e4m3(vals), codes)   # -0 keeps its sign code 0x80


def test_encode_midpoints_to_even_and_matches_torch():
    pos = np.arange(0, 0x7F, dtype=np.uint8)                  # 0 .. 448
    v = oracle.e4m3_to_f64(pos)
    mid = (v[:-1] + v[1:]) / 2                                # exact midpoints
    got = oracle.f64_to_e4m3(mid)
    even = np.where(pos[:-1] % 2 == 0, pos[:-1], pos[1:])     # the code with an even mantissa
    assert np.array_equal(got, even)
    assert np.array_equal(got, _torch_encode_f32(mid.astype(np.float32)))
    rng = np.random.default_rng(0)
    x = (rng.uniform(-448, 448, 20000) * rng.choice([1, 2.0 ** -5, 2.0 ** -9], 20000))
    x = x.astype(np.float32)
    assert np.array_equal(oracle.f64_to_e4m3(x.astype(np.float64)), _torch_encode_f32(x))


def test_pow2_scale_exponent():
    rng = np.random.default_rng(1)
    for a in np.exp(rng.uniform(np.log(1e-6), np.log(1e6), 2000)):
        e = oracle.pow2_scale_exp(a)
        assert a <= 448 * 2.0 ** e and a > 448 * 2.0 ** (e - 1)
    for j in range(-20, 21):
        assert oracle.pow2_scale_exp(448 * 2.0 ** j) == j
    assert oracle.pow2_scale_exp(0.0) == 0


def test_quantize_error_bound():
    rng = np.random.default_rng(2)
    x = oracle.f64_to_bf16(rng.standard_normal((300, D)) * rng.choice([1e-3, 1, 30], (300, 1)))
    codes, exps = oracle.quantize_e4m3(x)
    xv = oracle.bf16_to_f64(x)
    deq = oracle.e4m3_to_f64(codes) * (2.0 ** exps)[:, None]
    scaled = np.abs(xv) / (2.0 ** exps)[:, None]
    assert scaled.max(axis=1).max() <= 448 and (scaled.max(axis=1) > 224).all()
    # half a code spacing: 2^-4 relative in the normal range, 2^-10 (scaled) below 2^-6
    bound = (2.0 ** exps)[:, None] * np.maximum(scaled * 2.0 ** -4, 2.0 ** -10)
    assert (np.abs(xv - deq) <= bound).all()


def _representable_row(rng, n):
    """bf16 vectors whose entries are E4M3 values (|v| <= 16) with one entry 256: scale 2^0,
    and the codes represent the vector exactly."""
    vals = oracle.e4m3_to_f64(np.arange(0, 0x60, dtype=np.uint8))   # 0 .. 15
    x = rng.choice(vals, (n, D)) * rng.choice([-1, 1], (n, D))
    x[:, 0] = 256.0
    return oracle.f64_to_bf16(x)


def test_fp8_scores_equal_bf16_scores_when_representable():
    rng = np.random.default_rng(3)
    L = 50
    k = _representable_row(rng, L)
    q = _representable_row(rng, H).reshape(1, H, D)
    w = oracle.f64_to_bf16(rng.standard_normal((1, H)))
    kc, ke = oracle.quantize_e4m3(k)
    assert (ke == 0).all()
    assert np.array_equal(oracle.e4m3_to_f64(kc), oracle.bf16_to_f64(k))
    f8 = oracle.rows_fp8(q, w, kc, ke, [0], [L - 1], topk=16, full=True)
    b16 = oracle.rows(q, w, k, [0], [L - 1], topk=16, full=True)
    assert np.array_equal(f8["full"][0], b16["full"][0])
    assert np.array_equal(f8["idx"], b16["idx"])


def test_fp8_scores_power_of_two_key_scaling():
    rng = np.random.default_rng(4)
    L = 40
    k = oracle.f64_to_bf16(rng.standard_normal((L, D)))
    q = oracle.f64_to_bf16(rng.standard_normal((1, H, D)))
    w = oracle.f64_to_bf16(rng.standard_normal((1, H)) * 0.3)
    kc, ke = oracle.quantize_e4m3(k)
    base = oracle.rows_fp8(q, w, kc, ke, [0], [L - 1], topk=8, full=True)["full"][0]
    j = np.arange(L) % 5 - 2                                  # scale key s by 2^j[s]
    k2 = oracle.f64_to_bf16(oracle.bf16_to_f64(k) * (2.0 ** j)[:, None])
    kc2, ke2 = oracle.quantize_e4m3(k2)
    assert np.array_equal(kc2, kc) and np.array_equal(ke2, ke + j)
    scaled = oracle.rows_fp8(q, w, kc2, ke2, [0], [L - 1], topk=8, full=True)["full"][0]
    assert np.array_equal(scaled, base * 2.0 ** j)


def test_fp8_scores_query_head_scales():
    """Each query head carries its own power-of-two scale 2^eq[h], folded into its head
    weight: with heads scaled by 2^j (j != 0, up and down) the FP8 row must still equal the
    bf16 row exactly, so a dropped or inverted 2^eq factor fails here."""
    rng = np.random.default_rng(5)
    L = 60
    k = _representable_row(rng, L)
    j = np.array([(h % 7) - 3 if (h % 7) != 3 else 4 for h in range(H)])   # -3..4, never 0
    assert (j != 0).all()
    q0 = oracle.bf16_to_f64(_representable_row(rng, H))
    q = oracle.f64_to_bf16(q0 * (2.0 ** j)[:, None]).reshape(1, H, D)
    assert np.array_equal(oracle.bf16_to_f64(q).reshape(H, D), q0 * (2.0 ** j)[:, None])
    qc, qe = oracle.quantize_e4m3(q.reshape(H, D))
    assert np.array_equal(qe, j)                                # the scale is 2^j per head
    w = oracle.f64_to_bf16(rng.standard_normal((1, H)))
    f8 = oracle.rows_fp8(q, w, *oracle.quantize_e4m3(k), [0], [L - 1], topk=16, full=True)
    b16 = oracle.rows(q, w, k, [0], [L - 1], topk=16, full=True)
    assert np.array_equal(f8["full"][0], b16["full"][0])
    # one head at a time: the head's contribution scales by exactly 2^j[h]
    for h in (0, 3, 10, 31):
        wh = np.zeros((1, H), np.uint16)
        wh[0, h] = oracle.f64_to_bf16(np.array([1.0]))[0]
        one = oracle.rows_fp8(q, wh, *oracle.quantize_e4m3(k), [0], [L - 1], topk=4, full=True)["full"][0]
        q_un = oracle.f64_to_bf16(q0).reshape(1, H, D)
        base = oracle.rows(q_un, wh, k, [0], [L - 1], topk=4, full=True)["full"][0]
        assert np.array_equal(one, base * 2.0 ** j[h])
