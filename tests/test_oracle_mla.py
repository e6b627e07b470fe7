"""Pins of the oracle's sparse MLA over the selected tokens, on the CPU.

The reading ("Qwen3.5-397B-A17B vs Kimi K3.1 Pro" page, gated-MLA row: 96 heads, 576 cached
values per token = a 512-dim latent and a 64-dim key slot, each query attending only to the
tokens its indexer selects): absorbed queries q~ [96][576]; head h's logit for selected token
s is scale * q~_h . kv[s]; the softmax runs over the selected tokens; the output is the
softmax-weighted sum of their 512-dim latents.  Each pin below is a closed form or a special
case that a plausible slip (a dropped term, a wrong sign or index, the value taken from the
wrong part of the row, a missing normalisation) breaks."""
import numpy as np
import pytest

import oracle
from oracle import MLA_KV, MLA_V

H = 4   # heads in the small cases (the function is per head)


def _bf(x):
    return oracle.f64_to_bf16(np.asarray(x, dtype=np.float64))


def _rand(rng, shape, s=1.0):
    return _bf(rng.standard_normal(shape) * s)


def _z(q, kv, rows, scale):
    """Logits of one query (all heads) against the given cache rows, in fp64."""
    return scale * oracle.bf16_to_f64(q) @ oracle.bf16_to_f64(kv[rows]).T


def test_single_token_returns_its_latent():
    rng = np.random.default_rng(0)
    q = _rand(rng, (3, H, MLA_KV))
    kv = _rand(rng, (50, MLA_KV))
    idx = np.array([[7], [0], [49]], np.int32)
    o, lse = oracle.sparse_mla(q, kv, idx, scale=0.1)
    for t in range(3):
        r = idx[t, 0]
        assert np.array_equal(o[t], np.broadcast_to(oracle.bf16_to_f64(kv[r, :MLA_V]), (H, MLA_V)))
        assert np.allclose(lse[t], _z(q[t], kv, [r], 0.1)[:, 0], rtol=0, atol=1e-12)


def test_equal_logits_average_the_latents():
    rng = np.random.default_rng(1)
    q = np.zeros((2, H, MLA_KV), np.uint16)           # every logit 0
    kv = _rand(rng, (40, MLA_KV))
    idx = np.array([[3, 5, 8, 13, 21], [0, 1, 2, -1, -1]], np.int32)
    o, lse = oracle.sparse_mla(q, kv, idx)
    for t, rows in enumerate([[3, 5, 8, 13, 21], [0, 1, 2]]):
        mean = oracle.bf16_to_f64(kv[rows, :MLA_V]).mean(axis=0)
        assert np.allclose(o[t], mean[None, :], rtol=0, atol=1e-12)
        assert np.allclose(lse[t], np.log(len(rows)), rtol=0, atol=1e-12)


def test_two_tokens_logistic_closed_form():
    # o = v2 + sigmoid(z1 - z2) (v1 - v2), lse = z2 + log(1 + exp(z1 - z2))
    rng = np.random.default_rng(2)
    q = _rand(rng, (1, H, MLA_KV), 0.2)
    kv = _rand(rng, (10, MLA_KV))
    idx = np.array([[4, 9]], np.int32)
    o, lse = oracle.sparse_mla(q, kv, idx, scale=0.5)
    z = _z(q[0], kv, [4, 9], 0.5)
    v1, v2 = oracle.bf16_to_f64(kv[4, :MLA_V]), oracle.bf16_to_f64(kv[9, :MLA_V])
    sig = 1.0 / (1.0 + np.exp(-(z[:, 0] - z[:, 1])))
    assert np.allclose(o[0], v2[None, :] + sig[:, None] * (v1 - v2)[None, :], rtol=0, atol=1e-10)
    assert np.allclose(lse[0], z[:, 1] + np.log1p(np.exp(z[:, 0] - z[:, 1])), rtol=0, atol=1e-10)
    # the key slot (dims 512..575) counts in the logit but not in the value
    kv2 = kv.copy()
    kv2[4, MLA_V:] = _bf(oracle.bf16_to_f64(kv[4, MLA_V:]) + 1.0)
    o2, _ = oracle.sparse_mla(q, kv2, idx, scale=0.5)
    assert not np.allclose(o2, o)
    z2 = _z(q[0], kv2, [4, 9], 0.5)
    sig2 = 1.0 / (1.0 + np.exp(-(z2[:, 0] - z2[:, 1])))
    assert np.allclose(o2[0], v2[None, :] + sig2[:, None] * (v1 - v2)[None, :], rtol=0, atol=1e-10)


def test_duplicate_selection_doubles_the_weight():
    rng = np.random.default_rng(3)
    q = _rand(rng, (1, H, MLA_KV), 0.2)
    kv = _rand(rng, (10, MLA_KV))
    o, lse = oracle.sparse_mla(q, kv, np.array([[4, 9, 4]], np.int32), scale=0.5)
    z = _z(q[0], kv, [4, 9], 0.5)
    v1, v2 = oracle.bf16_to_f64(kv[4, :MLA_V]), oracle.bf16_to_f64(kv[9, :MLA_V])
    sig = 1.0 / (1.0 + np.exp(-(z[:, 0] + np.log(2.0) - z[:, 1])))
    assert np.allclose(o[0], v2[None, :] + sig[:, None] * (v1 - v2)[None, :], rtol=0, atol=1e-10)


def test_large_scale_selects_the_argmax():
    rng = np.random.default_rng(4)
    q = _rand(rng, (2, H, MLA_KV))
    kv = _rand(rng, (64, MLA_KV))
    idx = rng.permutation(64)[:32].astype(np.int32).reshape(2, 16)
    o, _ = oracle.sparse_mla(q, kv, idx, scale=1e6)
    for t in range(2):
        z = _z(q[t], kv, idx[t], 1.0)
        best = idx[t][np.argmax(z, axis=1)]
        assert np.array_equal(o[t], oracle.bf16_to_f64(kv[best, :MLA_V]))


def test_order_padding_offsets_and_empty_rows():
    rng = np.random.default_rng(5)
    q = _rand(rng, (3, H, MLA_KV), 0.1)
    kv = _rand(rng, (300, MLA_KV))
    idx = np.array([[1, 50, 99, 7], [7, 99, 1, 50], [-1, -1, -1, -1]], np.int32)
    o, lse = oracle.sparse_mla(q[[0, 0, 2]], kv, idx)
    assert np.allclose(o[0], o[1], rtol=0, atol=1e-12) and np.allclose(lse[0], lse[1], atol=1e-12)
    assert np.all(o[2] == 0) and np.all(np.isneginf(lse[2]))
    # -1 entries are skipped
    o2, lse2 = oracle.sparse_mla(q[[0]], kv, np.array([[1, -1, 50, -1, 99, 7]], np.int32))
    assert np.allclose(o2[0], o[0], rtol=0, atol=1e-12)
    # row offsets: idx relative to row0
    o3, _ = oracle.sparse_mla(q[[0]], kv, np.array([[1 - 1, 50 - 1, 99 - 1, 7 - 1]], np.int32),
                              row0=np.array([1], np.int64))
    assert np.allclose(o3[0], o[0], rtol=0, atol=1e-12)


def test_shift_invariance_through_the_key_slot():
    # adding c to every selected key slot (the same vector) adds scale * q_slot . c to every
    # logit of a head: the output is unchanged and lse moves by exactly that amount
    rng = np.random.default_rng(6)
    q = _rand(rng, (1, H, MLA_KV), 0.1)
    kv = _rand(rng, (20, MLA_KV))
    rows = np.array([[2, 3, 5, 7, 11, 13]], np.int32)
    o, lse = oracle.sparse_mla(q, kv, rows, scale=0.3)
    kv2 = kv.copy()
    kv2[:, MLA_V:] = 0
    kv3 = kv2.copy()
    kv3[:, MLA_V] = _bf([1.0])[0]                     # the slot dim 512 set to 1 on every row
    o2, lse2 = oracle.sparse_mla(q, kv2, rows, scale=0.3)
    o3, lse3 = oracle.sparse_mla(q, kv3, rows, scale=0.3)
    assert np.allclose(o3, o2, rtol=0, atol=1e-12)
    assert np.allclose(lse3 - lse2, 0.3 * oracle.bf16_to_f64(q[0, :, MLA_V]), rtol=0, atol=1e-12)
    assert not np.allclose(o2, o)                       # the slot did matter before
