"""Parity gates between a device result and the fp64 oracle.

bf16 path: max |o - o*| <= 2e-2 and mean |o - o*| <= 2e-3 over every element
(the stated tolerance for bf16 inputs with fp32 accumulation), plus a relative
Frobenius gate ||o - o*|| / ||o*|| <= 1e-2 so that an all-zero or mean-pooled
output cannot pass on small-magnitude outputs.  fp32 path: max-abs <= 1e-4.
LSE (natural log) is checked to 2e-2 absolute on bf16 and 1e-4 on fp32.
"""
import numpy as np

BF16_GATES = {"max_abs": 2e-2, "mean_abs": 2e-3, "rel_fro": 1e-2}
F32_GATES = {"max_abs": 1e-4, "mean_abs": 1e-5, "rel_fro": 1e-4}


def gates_for(dtype):
    return BF16_GATES if dtype == "bf16" else F32_GATES


def error_stats(out, ref):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = out - ref
    return {
        "max_abs": float(np.abs(d).max()) if d.size else 0.0,
        "mean_abs": float(np.abs(d).mean()) if d.size else 0.0,
        "rel_fro": float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)) if d.size else 0.0,
        "finite": bool(np.isfinite(out).all()),
    }


def passes(stats, gates):
    return stats["finite"] and all(stats[k] <= gates[k] for k in gates)


def assert_gates(out, ref, dtype, what=""):
    st = error_stats(out, ref)
    g = gates_for(dtype)
    assert passes(st, g), f"{what}: {st} vs gates {g}"
    return st


# ---------------------------------------------------------------- reduced-precision (SR_MX) gate
# The reduced-precision kernel computes attention over exactly the oracle's dequantized
# operands (MXFP6 q and k, FP8 v: the codes are bit-identical, checked separately), with one
# rounding the definition does not have: the probabilities are rounded to FP8 E4M3 (nearest
# even) before the P.V product, as p * 2^MX_PSHIFT relative to a running max that lags the
# true row max by at most 2 (log2), and the row sum is that of the rounded values.  With the
# exact normalised weights w_j of a row (fp64, over its visible keys) the rounded weights
# differ by at most
#     delta_j = min(w_j, max(2^-4 w_j, 2^-(10 + MX_PSHIFT) max_j w_j))
# (half an ulp of 3 mantissa bits on the normal range; half the smallest subnormal spacing
# 2^-9 of the scaled values below it, scaled by a max at most the true one).  Since
# sum_j w_j (v_j - o) = 0, the normalised result o' = sum w~_j v_j / sum w~_j satisfies
#     |o' - o| = |sum (w~_j - w_j)(v_j - o)| / sum w~_j <= (sum delta_j |v_j| + |o| sum delta_j) / (1 - sum delta_j)
# per feature.  Added: the matrix unit's accumulation of FP8 products (measured below 2e-4
# of sum |p v| per instruction; 4e-4 allowed), the bf16 rounding of the output (2^-9
# relative; 2^-8 allowed), fp32 arithmetic (the 1.02 factor and 1e-6).  The log-sum-exp
# changes by at most -ln(1 - sum delta) (+ the same accumulation term).
MX_PSHIFT = 6


def mx_bounds(w, v, o):
    """w [R, N] exact normalised weights, v [N, D] dequantized values, o [R, D] exact output
    (fp64) -> (per-element output bound [R, D], per-row lse bound [R])."""
    w = np.asarray(w, dtype=np.float64)
    av = np.abs(np.asarray(v, dtype=np.float64))
    ao = np.abs(np.asarray(o, dtype=np.float64))
    wmax = w.max(axis=1, keepdims=True)
    delta = np.minimum(w, np.maximum(2.0 ** -4 * w, 2.0 ** -(10 + MX_PSHIFT) * wmax))
    sd = delta.sum(axis=1, keepdims=True)
    assert (sd < 0.5).all(), "bound undefined: the rounding could remove half of the weight"
    b_o = 1.02 * (delta @ av + sd * ao) / (1.0 - sd) + 4e-4 * (w @ av) + 2.0 ** -8 * ao + 1e-6
    b_l = 1.02 * -np.log1p(-sd[:, 0]) + 4e-4 + 1e-6
    return b_o, b_l


def assert_mx(out, lse, o_ref, l_ref, b_o, b_l, what=""):
    """Every output element and lse value within its bound; returns the worst ratio err / bound."""
    out = np.asarray(out, dtype=np.float64)
    err_o = np.abs(out - o_ref)
    err_l = np.abs(np.asarray(lse, dtype=np.float64) - l_ref)
    assert np.isfinite(out).all(), what
    bad = err_o > b_o
    assert not bad.any(), (what, int(bad.sum()), float(err_o.max()), float((err_o / b_o).max()))
    assert (err_l <= b_l).all(), (what, float(err_l.max()), float((err_l / b_l).max()))
    return float((err_o / b_o).max()), float((err_l / b_l).max())
