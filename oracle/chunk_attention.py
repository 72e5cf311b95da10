"""One attention call of the current chunk over the oracle's cache model.

Visible set of current-chunk query i, with block b(i) = floor(i / causal_block):
  every persistent token of the call's bank, every token of the history chunks
  in the window, and the current-chunk tokens j with floor(j / causal_block) <= b(i).
(Prefix and window: project page "3.1.2 Historical Context and Temporal
Consistency"; per-step bank: "3.3 Inference Acceleration and End-to-End
Deployment".  The causal block inside the chunk is the whole chunk for
plain video chunks -- attention inside the window is bidirectional -- and one
latent frame for the frame-aligned semantic-reference layout, read as: a
frame's video and semantic tokens share one block; see the design notes.)
Queries are the current chunk's own tokens: row i is current token i.
"""
import numpy as np

from .attention import masked_attention, widen


def current_block_mask(rows, n_cur, causal_block):
    """bool [len(rows), n_cur]: current key j visible to query row i."""
    rows = np.asarray(rows)
    j = np.arange(n_cur)
    return (j[None, :] // causal_block) <= (rows[:, None] // causal_block)


def chunk_attention(cache, bank, q, scale, causal_block, dtype, heads=None, rows=None, row_block=2048):
    """q [n][H][D] storage array of the current chunk -> (o [len(rows)][len(heads)][D], lse [len(heads)][len(rows)]) fp64."""
    k, v, n_fixed = cache.sequence(bank)
    n_cur = k.shape[0] - n_fixed
    if q.shape[0] != n_cur:
        raise ValueError("queries are the current chunk's tokens")
    n_heads = q.shape[1]
    heads = list(range(n_heads)) if heads is None else list(heads)
    rows = np.arange(n_cur) if rows is None else np.asarray(rows)
    o = np.zeros((len(rows), len(heads), v.shape[2]))
    lse = np.zeros((len(heads), len(rows)))
    for hi, h in enumerate(heads):
        kh = widen(k[:, h, :], dtype)
        vh = widen(v[:, h, :], dtype)
        for r0 in range(0, len(rows), row_block):
            rb = rows[r0:r0 + row_block]
            qh = widen(q[rb, h, :], dtype)
            vis = np.concatenate([np.ones((len(rb), n_fixed), dtype=bool),
                                  current_block_mask(rb, n_cur, causal_block)], axis=1)
            ob, lb = masked_attention(qh, kh, vh, vis, scale)
            o[r0:r0 + len(rb), hi, :] = ob
            lse[hi, r0:r0 + len(rb)] = lb
    return o, lse
