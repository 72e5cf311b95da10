"""Masked scaled-dot-product attention in fp64: the definition the kernel must reach.

For one head, query row i and the set S(i) of keys visible to it:
    s_j  = scale * sum_d q_{i,d} k_{j,d}
    m    = max_{j in S(i)} s_j
    w_j  = exp(s_j - m)             (j in S(i)), 0 otherwise
    l    = sum_j w_j
    o_i  = sum_j w_j v_j / l
    lse  = m + ln l
This is softmax attention over the visible keys (project page "3.1.2 Historical
Context and Temporal Consistency": attention inside the window is bidirectional,
the moving rows attend to the whole window).  Subtracting m only conditions the
exponentials; it does not change o or lse.
"""
import numpy as np


def widen(x, dtype):
    """Storage values -> fp64.  bf16 arrives as uint16 bit patterns and widens exactly."""
    a = np.asarray(x)
    if dtype == "bf16":
        assert a.dtype == np.uint16
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        assert a.dtype == np.float32
        return a.astype(np.float64)
    raise ValueError(dtype)


def masked_attention(q, k, v, visible, scale, return_probs=False):
    """q [Nq, D], k [Nk, D], v [Nk, Dv] (fp64), visible bool [Nq, Nk] -> (o [Nq, Dv], lse [Nq]).

    Every row must see at least one key."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    visible = np.asarray(visible, dtype=bool)
    if not visible.any(axis=1).all():
        raise ValueError("a query row sees no key")
    s = scale * (q @ k.T)
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)                       # exp(-inf) = 0 on hidden keys
    l = w.sum(axis=1, keepdims=True)
    o = (w @ v) / l
    lse = m[:, 0] + np.log(l[:, 0])
    if return_probs:
        return o, lse, w / l
    return o, lse
