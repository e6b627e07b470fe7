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


def bf16_ulp(v):
    """Spacing of bf16 values at |v| (normal range)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def projection_bounds(A_bits, W_bits):
    """(exact fp64 product, deterministic fp32-summation error bound) of A @ W.

    For a K-term sum of exact products accumulated in fp32 in any order the error is at
    most (K - 1) * u * sum_i |a_i w_i| (u = 2^-24), to first order."""
    from oracle import bf16_to_f64
    A = bf16_to_f64(A_bits)
    W = bf16_to_f64(W_bits)
    K = A.shape[1]
    return A @ W, (K - 1) * U32 * (np.abs(A) @ np.abs(W))


def assert_bf16_within(g_bits, exact, err, name):
    """GPU bf16 result within err + one bf16 ulp of the exact value; returns the fraction of
    elements that differ from the correctly rounded value."""
    from oracle import bf16_to_f64, f64_to_bf16
    g = bf16_to_f64(g_bits).reshape(exact.shape)
    bound = err + bf16_ulp(exact)
    bad = np.abs(g - exact) > bound
    assert not bad.any(), f"{name}: {bad.sum()} elements outside the fp32 accumulation bound"
    return float((f64_to_bf16(exact) != g_bits.reshape(exact.shape)).mean())


def check_row_e2e(t, g_idx, g_sc, ref_e2e, r, ref_sw, r_sw, topk):
    """End-to-end row check: GPU result against the oracle run on its own projections.

    The GPU's bf16 projections may differ from the oracle's by one ulp where the exact
    product lies within the fp32 accumulation error of a rounding boundary.  Those input
    differences move each score by exactly |I_sw - I_e2e| (both fp64 oracle scores: on the
    GPU's projections and on the oracle's), which is added to the per-key tolerance."""
    n = min(topk, t + 1)
    g = np.asarray(g_idx)[:n]
    I = ref_e2e["full"][r]
    shift = np.abs(ref_sw["full"][r_sw] - I)
    tol = 1e-3 * ref_e2e["maxabs"][r] + 1e-5 + shift
    if g_sc is not None:
        err = np.abs(np.asarray(g_sc)[:n].astype(np.float64) - I[g])
        bad = err > tol[g]
        assert not bad.any(), f"row {t}: end-to-end score error {err[bad].max()} beyond tolerance"
    o = ref_e2e["idx"][r][:n]
    tau = ref_e2e["tau"][r]
    for s in set(g.tolist()) ^ set(o.tolist()):
        assert abs(I[s] - tau) <= tol[s] + shift.max(), \
            f"row {t}: index {s} differs with |I - tau| = {abs(I[s] - tau)}"
