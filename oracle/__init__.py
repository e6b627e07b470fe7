"""CPU oracle of the DSA lightning indexer forward pass -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library path never does, and it
shares no code with the HIP implementation.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over rows); this
module only marshals numpy arrays into it.  What it follows, from the
archdiff.com compare pages on Kimi K3.1 Pro (component tables):
  * sparse-attention row: q = c_q W_q (1,536 -> 4,096 = 32 heads x 128),
    k = LayerNorm(x W_k) (7,168 -> 128, one key shared by all heads),
    w = x W_w (7,168 -> 32), I = sum_h w_h ReLU(q_h . k), top 2,048 per query;
  * QK-norm row: the LayerNorm is on the indexer key;
  * RoPE row ("Kimi K3.1 Pro vs Gemma 4 31B" page): no rotary step in the indexer;
  * long-context row (same page): the whole prefix is scored.
The DeepSeek-V3.2-shaped indexer (64 heads, rotary step on 64 of the 128 dims) and the sparse
MLA over the selected tokens are at the end of this module.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_LIB names another build of oracle.c (build_sanitized()); the default is liboracle.so.
_SO_DEFAULT = os.path.join(_HERE, "liboracle.so")
_SO = os.environ.get("ORACLE_LIB") or _SO_DEFAULT
SO_SAN = os.path.join(_HERE, "_san", "liboracle.so")

H, D, QLAT, QOUT, HIDDEN, TOPK = 32, 128, 1536, 4096, 7168, 2048


def build(force=False):
    so = _SO_DEFAULT
    if force or not os.path.exists(so) or os.path.getmtime(so) < os.path.getmtime(_SRC):
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp",
                               "-fPIC", "-shared", _SRC, "-o", so + ".tmp", "-lm"])
        os.replace(so + ".tmp", so)


def build_sanitized():
    """oracle.c with gcc's AddressSanitizer and UndefinedBehaviorSanitizer, into _san/; load it
    with ORACLE_LIB in a process that preloads gcc's libasan and libubsan."""
    os.makedirs(os.path.dirname(SO_SAN), exist_ok=True)
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC",
                           "-shared", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", _SRC, "-o", SO_SAN, "-lm"])
    return SO_SAN


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        vp, i64, i32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.oracle_param_count.restype = i64
        L.oracle_param_count.argtypes = []
        L.oracle_num_threads.restype = i32
        L.oracle_num_threads.argtypes = []
        L.oracle_dims.restype = i32
        L.oracle_dims.argtypes = [vp]
        L.oracle_bf16_to_f64.restype = f64
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f64_to_bf16.restype = ctypes.c_uint16
        L.oracle_f64_to_bf16.argtypes = [f64]
        L.oracle_f64_to_bf16_array.restype = None
        L.oracle_f64_to_bf16_array.argtypes = [vp, i64, vp]
        L.oracle_linear_f64.restype = None
        L.oracle_linear_f64.argtypes = [vp, i64, vp, i64, i64, i64, vp]
        L.oracle_layernorm_f64.restype = None
        L.oracle_layernorm_f64.argtypes = [vp, i64, vp, vp, f64, vp]
        L.oracle_project.restype = None
        L.oracle_project.argtypes = [vp, i64, vp, i64, vp, vp, vp, vp, vp, f64, i64, vp, vp, vp]
        L.oracle_scores.restype = None
        L.oracle_scores.argtypes = [vp, vp, vp, i64, i32, i32, vp]
        L.oracle_topk.restype = None
        L.oracle_topk.argtypes = [vp, i64, i32, vp, vp, vp, vp]
        L.oracle_rows.restype = None
        L.oracle_rows.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.oracle_e4m3_to_f64.restype = f64
        L.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        L.oracle_f64_to_e4m3.restype = ctypes.c_uint8
        L.oracle_f64_to_e4m3.argtypes = [f64]
        L.oracle_pow2_scale_exp.restype = i32
        L.oracle_pow2_scale_exp.argtypes = [f64]
        L.oracle_quantize_e4m3.restype = None
        L.oracle_quantize_e4m3.argtypes = [vp, i64, i32, vp, vp]
        L.oracle_sparse_mla.restype = None
        L.oracle_sparse_mla.argtypes = [vp, vp, vp, vp, i64, i32, i32, f64, vp, vp]
        L.oracle_rows_fp8.restype = None
        L.oracle_rows_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, vp, vp, vp, vp,
                                      vp, vp]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ---------------------------------------------------------------- numbers
def bf16_to_f64(b):
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16(x):
    x = _c(x, np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_f64_to_bf16_array(_p(x), x.size, _p(out))
    return out


def param_count():
    return int(lib().oracle_param_count())


def num_threads():
    return int(lib().oracle_num_threads())


def dims():
    d = np.zeros(6, dtype=np.int32)
    lib().oracle_dims(_p(d))
    return dict(zip(("heads", "dim", "qlat", "qout", "hidden", "topk"), d.tolist()))


# ---------------------------------------------------------------- projections
def linear_f64(A, W):
    A = _c(A, np.uint16)
    W = _c(W, np.uint16)
    rows, n_in = A.shape
    n_out = W.shape[1]
    out = np.empty((rows, n_out), dtype=np.float64)
    lib().oracle_linear_f64(_p(A), n_in, _p(W), n_in, n_out, rows, _p(out))
    return out


def layernorm_f64(a, gamma, beta, eps):
    a = _c(a, np.float64)
    g = _c(gamma, np.uint16)
    b = _c(beta, np.uint16)
    out = np.empty_like(a)
    for r in range(a.shape[0]):
        lib().oracle_layernorm_f64(a[r].ctypes.data, a.shape[1], _p(g), _p(b), float(eps),
                                   out[r].ctypes.data)
    return out


def project(x, c_q, Wt, want=("q", "k", "w")):
    """q [T,32,128], k [T,128], w [T,32] (bf16 patterns) of one indexer layer."""
    T = (x if x is not None else c_q).shape[0]
    x = None if x is None else _c(x, np.uint16)
    c_q = None if c_q is None else _c(c_q, np.uint16)
    q = np.empty((T, H, D), np.uint16) if "q" in want else None
    k = np.empty((T, D), np.uint16) if "k" in want else None
    w = np.empty((T, H), np.uint16) if "w" in want else None
    lib().oracle_project(_p(x), HIDDEN, _p(c_q), QLAT, _p(_c(Wt["W_q"], np.uint16)),
                         _p(_c(Wt["W_k"], np.uint16)), _p(_c(Wt["W_w"], np.uint16)),
                         _p(_c(Wt["gamma"], np.uint16)), _p(_c(Wt["beta"], np.uint16)),
                         float(Wt["eps"]), T, _p(q), _p(k), _p(w))
    return q, k, w


# ---------------------------------------------------------------- scores and top-k
def scores(q_row, w_row, k, n=None):
    """I[s] for s < n of one query row; q_row [H,D], w_row [H], k [>=n, D] (bf16 patterns)."""
    q_row = _c(q_row, np.uint16)
    w_row = _c(w_row, np.uint16)
    k = _c(k, np.uint16)
    Hh, Dd = q_row.shape
    n = k.shape[0] if n is None else n
    out = np.empty(n, dtype=np.float64)
    lib().oracle_scores(_p(q_row), _p(w_row), _p(k), n, Hh, Dd, _p(out))
    return out


def topk(I, k=TOPK):
    I = _c(I, np.float64)
    idx = np.empty(k, dtype=np.int32)
    sc = np.empty(k, dtype=np.float64)
    tau = np.zeros(1)
    m = np.zeros(1)
    lib().oracle_topk(_p(I), I.size, k, _p(idx), _p(sc), _p(tau), _p(m))
    return idx, sc, float(tau[0]), float(m[0])


def rows(q_rows, w_rows, k, k_off, t, topk=TOPK, full=False):
    """Score and select a batch of query rows.

    q_rows [R,H,D], w_rows [R,H]; row r scores keys k[k_off[r] : k_off[r] + t[r] + 1].
    Rows are handed to OpenMP longest first.  Returns dict(idx [R,topk] int32,
    score [R,topk] f64, tau [R], maxabs [R], full (list of per-row score vectors or None)).
    """
    q_rows = _c(q_rows, np.uint16)
    w_rows = _c(w_rows, np.uint16)
    k = _c(k, np.uint16)
    k_off = _c(k_off, np.int64)
    t = _c(t, np.int64)
    R = t.size
    Hh, Dd = q_rows.shape[1], q_rows.shape[2]
    order = np.argsort(-t, kind="stable")
    qo, wo, ko, to = (_c(q_rows[order], np.uint16), _c(w_rows[order], np.uint16),
                      _c(k_off[order], np.int64), _c(t[order], np.int64))
    idx = np.empty((R, topk), np.int32)
    sc = np.empty((R, topk), np.float64)
    tau = np.empty(R)
    m = np.empty(R)
    fbuf = foff = None
    if full:
        foff = np.zeros(R, dtype=np.int64)
        foff[1:] = np.cumsum(to + 1)[:-1]
        fbuf = np.empty(int((to + 1).sum()), dtype=np.float64)
    lib().oracle_rows(_p(qo), _p(wo), _p(k), _p(ko), _p(to), R, Hh, Dd, topk, _p(idx), _p(sc),
                      _p(tau), _p(m), _p(fbuf), _p(foff))
    inv = np.empty(R, dtype=np.int64)
    inv[order] = np.arange(R)
    out = dict(idx=idx[inv], score=sc[inv], tau=tau[inv], maxabs=m[inv], full=None)
    if full:
        vec = [fbuf[foff[j]:foff[j] + to[j] + 1] for j in range(R)]
        out["full"] = [vec[inv[r]] for r in range(R)]
    return out


def prefill_rows(q, k, w, row_ids, topk=TOPK, full=False):
    """Rows of one causal sequence: q [T,H,D], k [T,D], w [T,H]."""
    row_ids = np.asarray(row_ids, dtype=np.int64)
    return rows(q[row_ids], w[row_ids], k, np.zeros_like(row_ids), row_ids, topk, full)


# ---------------------------------------------------------------- FP8 (OCP E4M3) key cache
def e4m3_to_f64(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    return np.array([lib().oracle_e4m3_to_f64(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def f64_to_e4m3(x):
    x = np.asarray(x, dtype=np.float64)
    return np.array([lib().oracle_f64_to_e4m3(float(v)) for v in x.ravel()], np.uint8).reshape(x.shape)


def pow2_scale_exp(amax):
    return int(lib().oracle_pow2_scale_exp(float(amax)))


def quantize_e4m3(x):
    """x [n, d] bf16 patterns -> (codes [n, d] uint8, exponents [n] int32): scale 2^e per row."""
    x = _c(x, np.uint16)
    n, d = x.shape
    codes = np.empty((n, d), np.uint8)
    exps = np.empty(n, np.int32)
    lib().oracle_quantize_e4m3(_p(x), n, d, _p(codes), _p(exps))
    return codes, exps


def rows_fp8(q_rows, w_rows, k_codes, k_exps, k_off, t, topk=TOPK, full=False):
    """FP8 decode rows: q_rows [R,H,D] bf16 (quantised here per head), w_rows [R,H] bf16,
    k_codes [*, D] uint8 with exponents k_exps; row r scores cache rows k_off[r] .. + t[r]."""
    q_rows = _c(q_rows, np.uint16)
    R, Hh, Dd = q_rows.shape
    qc, qe = quantize_e4m3(q_rows.reshape(R * Hh, Dd))
    qc = _c(qc.reshape(R, Hh, Dd), np.uint8)
    qe = _c(qe.reshape(R, Hh), np.int32)
    w_rows = _c(w_rows, np.uint16)
    k_codes = _c(k_codes, np.uint8)
    k_exps = _c(k_exps, np.int32)
    k_off = _c(k_off, np.int64)
    t = _c(t, np.int64)
    idx = np.empty((R, topk), np.int32)
    sc = np.empty((R, topk), np.float64)
    tau = np.empty(R)
    m = np.empty(R)
    fbuf = foff = None
    if full:
        foff = np.zeros(R, dtype=np.int64)
        foff[1:] = np.cumsum(t + 1)[:-1]
        fbuf = np.empty(int((t + 1).sum()), dtype=np.float64)
    lib().oracle_rows_fp8(_p(qc), _p(qe), _p(w_rows), _p(k_codes), _p(k_exps), _p(k_off), _p(t), R,
                          Hh, Dd, topk, _p(idx), _p(sc), _p(tau), _p(m), _p(fbuf), _p(foff))
    out = dict(idx=idx, score=sc, tau=tau, maxabs=m, full=None)
    if full:
        out["full"] = [fbuf[foff[j]:foff[j] + t[j] + 1] for j in range(R)]
    return out


# ---------------------------------------------------------------- sparse MLA consumer
MLA_HEADS, MLA_KV, MLA_V = 96, 576, 512


def sparse_mla(q, kv, idx, row0=None, scale=1.0 / np.sqrt(192.0)):
    """Sparse MLA over the selected tokens (gated-MLA row of the "Qwen3.5-397B-A17B vs Kimi
    K3.1 Pro" page, absorbed-query reading): q [T,H,576] bf16, kv [*,576] bf16, idx [T,K] int32
    (-1 = none), row0 [T] or None.  Returns (o [T,H,512] f64, lse [T,H] f64)."""
    q = _c(q, np.uint16)
    T, Hh, Dk = q.shape
    assert Dk == MLA_KV
    kv = _c(kv, np.uint16)
    idx = _c(idx, np.int32)
    K = idx.shape[1]
    r0 = None if row0 is None else _c(row0, np.int64)
    o = np.empty((T, Hh, MLA_V), np.float64)
    lse = np.empty((T, Hh), np.float64)
    lib().oracle_sparse_mla(_p(q), _p(kv), _p(idx), _p(r0), T, Hh, K, float(scale), _p(o), _p(lse))
    return o, lse


# ---------------------------------------------------------------- DeepSeek-V3.2-shaped indexer
# The sparse-attention row of the "Qwen3.5-397B-A17B vs Kimi K3.1 Pro" page gives DeepSeek-
# V3.2's indexer 64 heads, and the RoPE row of the "Kimi K3.1 Pro vs Gemma 4 31B" page says
# it rotates 64 of its 128 dims.  Read here as the K3.1 indexer above with those two changes:
# q = c_q W_q (1,536 -> 8,192 = 64 heads x 128), k = LayerNorm(x W_k) (7,168 -> 128),
# w = x W_w (7,168 -> 64), I = sum over the 64 heads; the rotary step turns dims (2i, 2i+1),
# i < 32, of every query head and of the key by the angle pos * theta^(-2i/64) (theta = 10^4),
# applied to the exact projection (for k after its LayerNorm), and the rotated vector is rounded
# to bf16 once, as the K3.1 projections are.  Dims 64..127 are not rotated.
V32_H, V32_QOUT, V32_ROT, V32_THETA = 64, 8192, 64, 10000.0


def rope_angles(pos, rot=V32_ROT, theta=V32_THETA):
    """Angles [len(pos), rot/2] in fp64: position times theta^(-2i/rot)."""
    i = np.arange(rot // 2, dtype=np.float64)
    return np.asarray(pos, dtype=np.float64)[:, None] * theta ** (-2.0 * i / rot)[None, :]


def rope_f64(v, pos, rot=V32_ROT, theta=V32_THETA):
    """The rotary step on v [T, ..., 128] (fp64 values) at positions pos [T]: returns fp64.

    Pair i of a vector, (v[2i], v[2i+1]), becomes (v[2i] c - v[2i+1] s, v[2i] s + v[2i+1] c)
    with c, s the cosine and sine of its angle; the dims past `rot` are copied."""
    v = np.asarray(v, dtype=np.float64)
    a = rope_angles(pos, rot, theta)
    shape = (v.shape[0],) + (1,) * (v.ndim - 2) + (rot // 2,)
    c, s = np.cos(a).reshape(shape), np.sin(a).reshape(shape)
    out = v.copy()
    x, y = v[..., 0:rot:2], v[..., 1:rot:2]
    out[..., 0:rot:2] = x * c - y * s
    out[..., 1:rot:2] = x * s + y * c
    return out


def project_v32(x, c_q, Wt, pos0=0, theta=V32_THETA, want=("q", "k", "w")):
    """q [T,64,128], k [T,128], w [T,64] (bf16 patterns) of the DeepSeek-V3.2-shaped indexer
    for tokens at positions pos0 .. pos0 + T - 1: the rotary step on the exact fp64 q and on the
    exact LayerNorm of the key, each result rounded to bf16 once."""
    T = (x if x is not None else c_q).shape[0]
    pos = pos0 + np.arange(T, dtype=np.int64)
    q = k = w = None
    if "q" in want:
        q = f64_to_bf16(rope_f64(linear_f64(c_q, Wt["W_q"]).reshape(T, V32_H, D), pos, theta=theta))
    if "k" in want:
        lin = linear_f64(x, Wt["W_k"])
        k = f64_to_bf16(rope_f64(layernorm_f64(lin, Wt["gamma"], Wt["beta"], Wt["eps"]), pos, theta=theta))
    if "w" in want:
        w = f64_to_bf16(linear_f64(x, Wt["W_w"]))
    return q, k, w
