"""The indexer workloads as seeded synthetic inputs (host numpy arrays).

Shapes follow the DSA indexer of Kimi K3.1 Pro (32 heads x 128 dims, query
latent 1,536, hidden 7,168, top 2,048).  ``var`` arguments are variances, so
N(0, 1/fan_in) weights have std 1/sqrt(fan_in) and N(0, 0.1) head weights have
std 0.316.  Every function takes the sizes as arguments so that tests can draw
the same distributions at smaller shapes.
"""
import numpy as np

from . import (BETA, CQ, GAMMA, K, KCACHE, Q, SEQLEN, W, WK, WQ, WW, X, normal_bf16,
               uniform_f64, uniform_int)

H, D, QLAT, QOUT, HIDDEN, TOPK = 32, 128, 1536, 4096, 7168, 2048
LN_EPS = 1e-6


def score_inputs(T, seed=0, layer=0):
    """Score + top-k only: q [T,32,128] ~N(0,1), k [T,128] ~N(0,1), w [T,32] ~N(0,0.1)."""
    return dict(q=normal_bf16((T, H, D), 0.0, 1.0, Q, layer, seed),
                k=normal_bf16((T, D), 0.0, 1.0, K, layer, seed),
                w=normal_bf16((T, H), 0.0, 0.1, W, layer, seed))


def chunk_inputs(prefix, C, seed=0, layer=0):
    """Chunked prefill: the queries and head weights of positions prefix .. prefix + C - 1
    and the keys of positions 0 .. prefix + C - 1, the same values as
    score_inputs(T)[...][prefix : prefix + C] (q, w) and [: prefix + C] (k) for any larger T."""
    return dict(q=normal_bf16((C, H, D), 0.0, 1.0, Q, layer, seed, first=prefix * H * D),
                k=normal_bf16((prefix + C, D), 0.0, 1.0, K, layer, seed),
                w=normal_bf16((C, H), 0.0, 0.1, W, layer, seed, first=prefix * H))


def layer_weights(layer=0, seed=0):
    """One indexer layer: W_q ~N(0,1/1536), W_k, W_w ~N(0,1/7168), gamma ~1+N(0,0.02), beta ~N(0,0.02)."""
    return dict(W_q=normal_bf16((QLAT, QOUT), 0.0, 1.0 / QLAT, WQ, layer, seed),
                W_k=normal_bf16((HIDDEN, D), 0.0, 1.0 / HIDDEN, WK, layer, seed),
                W_w=normal_bf16((HIDDEN, H), 0.0, 1.0 / HIDDEN, WW, layer, seed),
                gamma=normal_bf16((D,), 1.0, 0.02, GAMMA, layer, seed),
                beta=normal_bf16((D,), 0.0, 0.02, BETA, layer, seed),
                eps=LN_EPS)


def layer_weights_v32(layer=0, seed=0):
    """One DeepSeek-V3.2-shaped indexer layer (64 heads): W_q [1536, 8192] ~N(0,1/1536), W_k
    [7168, 128] and W_w [7168, 64] ~N(0,1/7168), gamma and beta as above.  Drawn from the
    streams of `layer_weights` at layer index 4096 + layer, so the two shapes never share
    values."""
    lv = 4096 + layer
    return dict(W_q=normal_bf16((QLAT, 2 * QOUT), 0.0, 1.0 / QLAT, WQ, lv, seed),
                W_k=normal_bf16((HIDDEN, D), 0.0, 1.0 / HIDDEN, WK, lv, seed),
                W_w=normal_bf16((HIDDEN, 2 * H), 0.0, 1.0 / HIDDEN, WW, lv, seed),
                gamma=normal_bf16((D,), 1.0, 0.02, GAMMA, lv, seed),
                beta=normal_bf16((D,), 0.0, 0.02, BETA, lv, seed),
                eps=LN_EPS)


def layer_activations(T, seed=0, layer=0):
    """Hidden state x [T,7168] and query latent c_q [T,1536], both ~N(0,1)."""
    return dict(x=normal_bf16((T, HIDDEN), 0.0, 1.0, X, layer, seed),
                c_q=normal_bf16((T, QLAT), 0.0, 1.0, CQ, layer, seed))


def decode_lengths(B, lo=32768, hi=131072, seed=0):
    """Cached key counts per sequence, uniform integers in [lo, hi] (own key included)."""
    return uniform_int(B, lo, hi, SEQLEN, 0, seed)


def decode_cache(lengths, seed=0):
    """Packed key cache [sum L, 128] bf16 ~N(0,1); row start[b] + L_b - 1 is left for the
    new token's projected key.  Returns (cache, start)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    start = np.zeros(len(lengths), dtype=np.int64)
    start[1:] = np.cumsum(lengths)[:-1]
    cache = normal_bf16((int(lengths.sum()), D), 0.0, 1.0, KCACHE, 0, seed)
    return cache, start


def varlen_lengths(B, lo=2048, hi=32768, seed=0):
    """L_b = floor(exp(U(ln lo, ln hi))) clamped to [lo, hi] (log-uniform lengths)."""
    u = uniform_f64(B, SEQLEN, 1, seed)
    L = np.floor(np.exp(np.log(lo) + u * (np.log(hi) - np.log(lo)))).astype(np.int64)
    return np.clip(L, lo, hi)


def cu_seqlens(lengths):
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    return cu
