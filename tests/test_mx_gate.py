"""The reduced-precision parity gate (gates.mx_bounds) against a simulation of the rounding it
accounts for, on the CPU.

The simulation takes the exact logits of the dequantized operands and does what the bound
assumes the kernel does: probabilities relative to a running max that lags the row max by
up to 2 (log2), scaled by 2^6, rounded to FP8 E4M3 (oracle.mx's encoder: nearest, ties to
even), then normalised by the sum of the rounded values.  The bound must hold for every
element, and it must be tight enough to reject the same kernel without the 2^6 scaling
(probabilities below 2^-10 of the max flushed to zero) on rows with a heavy low tail.
"""
import numpy as np
import pytest

import gates
import oracle
from oracle import mx as omx

LOG2E = 1.4426950408889634


def simulated(q, k, v, scale, lag, pshift):
    s = scale * (q @ k.T) * LOG2E                       # log2 units
    m_s = s.max(axis=1, keepdims=True) - lag[:, None]     # stale running max
    qv = np.exp2(s - m_s + pshift)
    assert qv.max() <= 448.0
    qr = omx.decode(omx.encode(qv, omx.E4M3), omx.E4M3)
    l = qr.sum(axis=1, keepdims=True)
    o = (qr @ v) / l
    lse = (m_s[:, 0] + np.log2(l[:, 0]) - pshift) / LOG2E
    return o, lse


@pytest.mark.parametrize("logit_std,n_keys,seed", [(1.0, 300, 1), (4.0, 2000, 2), (0.05, 5000, 3), (25.0, 700, 4)])
def test_bound_holds_on_simulated_rounding(logit_std, n_keys, seed):
    r = np.random.default_rng(seed)
    D, R = 64, 40
    q = omx.mxfp6_values(r.standard_normal((R, D)))
    k = omx.mxfp6_values(r.standard_normal((n_keys, D)) * logit_std)
    v = omx.fp8_values(r.standard_normal((n_keys, D)) + r.uniform(-2, 2, (1, D)))
    scale = 1.0 / np.sqrt(D)
    o, lse, w = oracle.masked_attention(q, k, v, np.ones((R, n_keys), bool), scale, return_probs=True)
    b_o, b_l = gates.mx_bounds(w, v, o)
    for lag in (np.zeros(R), np.full(R, 1.999), r.uniform(0, 2, R)):
        o2, l2 = simulated(q, k, v, scale, lag, gates.MX_PSHIFT)
        assert (np.abs(o2 - o) <= b_o).all(), float((np.abs(o2 - o) / b_o).max())
        assert (np.abs(l2 - lse) <= b_l).all()


def test_bound_rejects_unscaled_probabilities():
    """A row whose weight sits mostly in a tail of keys 2^-11 below the max: without the 2^6
    shift the kernel would flush that tail and miss the bound."""
    r = np.random.default_rng(7)
    D, n = 64, 4000
    q = np.zeros((1, D))
    q[0, 0] = 1.0
    k = np.zeros((n, D))
    k[0, 0] = 11.0 / LOG2E               # one key 11 (log2) above the rest
    v = omx.fp8_values(r.standard_normal((n, D)) + 1.0)
    o, lse, w = oracle.masked_attention(q, k, v, np.ones((1, n), bool), 1.0, return_probs=True)
    b_o, b_l = gates.mx_bounds(w, v, o)
    o_ok, _ = simulated(q, k, v, 1.0, np.zeros(1), gates.MX_PSHIFT)
    assert (np.abs(o_ok - o) <= b_o).all()
    o_bad, l_bad = simulated(q, k, v, 1.0, np.zeros(1), 0)
    assert (np.abs(o_bad - o) > b_o).any() and (np.abs(l_bad - lse) > b_l).any()
