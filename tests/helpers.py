"""Shared test plumbing: host <-> device bf16 arrays and the parity rule.

Parity rule for one query row t (scores in fp32 on the GPU, fp64 in the oracle):
  tol_t = 1e-3 * max_s |I_oracle[t, s]| + 1e-5
  * the GPU returns exactly min(topk, t+1) distinct indices in [0, t], ascending, then -1;
  * every returned score is within tol_t of the oracle score of the same index, and the
    padding scores are -inf;
  * every index in the symmetric difference of the GPU and oracle sets has an oracle score
    within tol_t of the row's topk-th oracle score (only near-ties may differ).
"""
import numpy as np
import torch


def to_dev(a, dev="cuda"):
    """uint16 bf16 patterns (numpy) -> torch.bfloat16 on the device."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def to_host(t):
    """torch.bfloat16 -> uint16 bf16 patterns (numpy)."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def weights_to_dev(Wt, dev="cuda"):
    d = {k: to_dev(v, dev) for k, v in Wt.items() if k != "eps"}
    d["eps"] = Wt["eps"]
    return d


def check_row(t, g_idx, g_sc, ref, r, topk, exact=False):
    """Check GPU row (g_idx [topk], g_sc [topk] or None) against oracle result row r.

    Returns the number of band-excused index differences."""
    n = min(topk, t + 1)
    g_idx = np.asarray(g_idx)
    assert np.all(g_idx[n:] == -1), f"row {t}: padding is not -1"
    g = g_idx[:n]
    assert np.all(g >= 0) and np.all(g <= t), f"row {t}: index out of [0, {t}]"
    assert np.all(np.diff(g) > 0), f"row {t}: indices not strictly ascending"
    I = ref["full"][r]
    o = ref["idx"][r][:n]
    tol = 1e-3 * ref["maxabs"][r] + 1e-5
    if g_sc is not None:
        g_sc = np.asarray(g_sc)
        err = np.abs(g_sc[:n].astype(np.float64) - I[g])
        assert err.max(initial=0.0) <= tol, f"row {t}: score error {err.max()} > tol {tol}"
        assert np.all(np.isneginf(g_sc[n:])), f"row {t}: padding score is not -inf"
        if exact:
            assert np.array_equal(g_sc[:n].astype(np.float64), I[g]), f"row {t}: scores not exact"
    diff = set(g.tolist()) ^ set(o.tolist())
    if exact:
        assert not diff, f"row {t}: selection differs: {sorted(diff)[:10]}"
    for s in diff:
        assert abs(I[s] - ref["tau"][r]) <= tol, \
            f"row {t}: index {s} differs with |I - tau| = {abs(I[s] - ref['tau'][r])} > {tol}"
    return len(diff)


# ------------------------------------------------------------------ projection tolerance
U32 = 2.0 ** -24   # unit roundoff of fp32
SIGMAS = 10.0      # radius of the projection error model, in standard deviations


def bf16_ulp(v):
    """Spacing of bf16 values at |v| (normal range)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _rne(x):
    from oracle import bf16_to_f64, f64_to_bf16
    return bf16_to_f64(f64_to_bf16(x))


def linear_exact(A_bits, W_bits):
    """(exact fp64 product A @ W, radius of the GPU's fp32 result around it).

    The products of bf16 values are exact in fp32; only the K - 1 additions round.  With
    rounding errors independent, of size at most u = 2^-24 relative (variance u^2/3), and
    zero-mean terms x_i = a_i w_i, the partial sums S_j have E[S_j^2] = sum_{i<=j} x_i^2 <=
    ||x||^2, so the accumulated error has standard deviation at most u sqrt(K/3) ||x||_2 in
    any summation order (a blocked order makes fewer roundings and only lowers it).  The
    radius is SIGMAS such deviations.  The deterministic worst case, (K - 1) u sum |x_i|, is
    about 50 times larger at these shapes and would admit almost any neighbouring bf16 value."""
    from oracle import bf16_to_f64
    A = bf16_to_f64(A_bits)
    W = bf16_to_f64(W_bits)
    K = A.shape[1]
    return A @ W, SIGMAS * U32 * np.sqrt(K / 3.0) * np.sqrt((A * A) @ (W * W))


def layernorm_exact(ea, ra, Wt):
    """(LayerNorm of the exact pre-norm values ea, radius of the GPU's fp32 result).

    To first order a pre-norm error d moves k_i by gamma_i / sigma (d_i - mean(d) -
    khat_i mean(khat d)), khat = (ea - mean) / sigma; |d_j| <= ra_j bounds that term.  The
    LayerNorm's own fp32 arithmetic adds a few u relative: 16 u (|k| + 1)."""
    import oracle
    ek = oracle.layernorm_f64(ea, Wt["gamma"], Wt["beta"], Wt["eps"])
    mu = ea.mean(axis=1, keepdims=True)
    sigma = np.sqrt(ea.var(axis=1, keepdims=True) + Wt["eps"])
    kh = np.abs(ea - mu) / sigma
    gam = np.abs(oracle.bf16_to_f64(Wt["gamma"]))[None, :]
    rk = gam / sigma * (ra + ra.mean(axis=1, keepdims=True)
                        + kh * (kh * ra).mean(axis=1, keepdims=True))
    return ek, rk + 16 * U32 * (np.abs(ek) + 1)


def key_exact(x_bits, Wt, chunk=8192):
    """linear_exact + layernorm_exact of the key projection, in row chunks."""
    e = np.empty((x_bits.shape[0], Wt["W_k"].shape[1]))
    r = np.empty_like(e)
    for a in range(0, x_bits.shape[0], chunk):
        ea, ra = linear_exact(x_bits[a:a + chunk], Wt["W_k"])
        e[a:a + chunk], r[a:a + chunk] = layernorm_exact(ea, ra, Wt)
    return e, r


def assert_bf16_within(g_bits, exact, err, name):
    """GPU bf16 result within err of the exact value (for values rounded twice, where err
    already carries the roundings)."""
    from oracle import bf16_to_f64
    g = bf16_to_f64(g_bits).reshape(exact.shape)
    bad = np.abs(g - exact) > err
    assert not bad.any(), f"{name}: {bad.sum()} elements outside the error bound"


def check_projection(g_bits, e, r, name):
    """The GPU's bf16 value of each element is the bf16 rounding of some fp32 value within r of
    the exact value e (so it lies in [rne(e - r), rne(e + r)]).  Returns the fraction of
    elements that differ from the correctly rounded rne(e)."""
    from oracle import bf16_to_f64
    g = bf16_to_f64(g_bits).reshape(e.shape)
    lo, hi = _rne(e - r), _rne(e + r)
    bad = ~((g >= lo) & (g <= hi))
    if bad.any():
        j = np.argwhere(bad)[0]
        raise AssertionError(f"{name}: {int(bad.sum())} elements outside the rounding radius, first "
                             f"at {tuple(j)}: gpu {g[tuple(j)]!r}, exact {e[tuple(j)]!r}, radius {r[tuple(j)]!r}")
    return float((g != _rne(e)).mean())


def flip_slack(o_bits, e, r):
    """How far the GPU's value of each element may lie from the oracle's bf16 value o_bits
    (the rounding of e): the largest |rne(f) - o| over |f - e| <= r; zero for every element not
    within r of a rounding boundary."""
    from oracle import bf16_to_f64
    o = bf16_to_f64(o_bits).reshape(e.shape)
    return np.maximum(_rne(e + r) - o, o - _rne(e - r))


def score_slack(q, dq, w, dw, k, dk):
    """Bound on the change of I[s] = sum_h w_h ReLU(q_h . k_s) when each element of q [H,D],
    w [H] and k [n,D] (fp64 values) moves by at most dq, dw, dk: with e_h = sum_i dq|k| + |q|dk
    + dq dk (ReLU is 1-Lipschitz), |dI| <= sum_h dw_h (ReLU(q_h . k) + e_h) + |w_h| e_h."""
    E = dq @ np.abs(k).T + np.abs(q) @ dk.T + dq @ dk.T
    d = np.maximum(q @ k.T, 0.0)
    return (dw[:, None] * (d + E) + np.abs(w)[:, None] * E).sum(axis=0)


def check_row_e2e(t, g_idx, g_sc, ref, r, topk, slack):
    """End-to-end row check: GPU result against the oracle run on its own projections.

    slack[s] (from score_slack on the oracle's projections and their flip_slack) bounds how
    far I[s] can move when the GPU's projections differ from the oracle's within their rounding
    radius, which check_projection verifies for every element this row reads.  Per key the
    tolerance is the parity rule's plus slack[s]; an index may differ between the two
    selections only if |I[s] - tau| is within its own tolerance plus the largest tolerance
    among the differing indices (the other side of the swap)."""
    n = min(topk, t + 1)
    g = np.asarray(g_idx)[:n]
    I = ref["full"][r]
    tol = 1e-3 * (ref["maxabs"][r] + slack.max(initial=0.0)) + 1e-5 + slack
    if g_sc is not None:
        err = np.abs(np.asarray(g_sc)[:n].astype(np.float64) - I[g])
        bad = err > tol[g]
        assert not bad.any(), f"row {t}: end-to-end score error {err[bad].max()} beyond tolerance"
    o = ref["idx"][r][:n]
    diff = np.array(sorted(set(g.tolist()) ^ set(o.tolist())), dtype=np.int64)
    if len(diff):
        far = np.abs(I[diff] - ref["tau"][r]) > tol[diff] + tol[diff].max()
        assert not far.any(), f"row {t}: index {diff[far][0]} differs beyond the band"
