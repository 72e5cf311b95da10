"""Page-literal window variant: attention of the moving rows and of the prefix rows.

Project page "3.1.2 Historical Context and Temporal Consistency": a window is a fixed
prefix (text/image conditioning, reference image, sink) followed by a moving part (the
recent history and the current chunk).  Attention inside the window is bidirectional; the
prefix attends only to itself and the moving part attends to the whole window.  With the
prefix cache only the recent history and the current chunk are recomputed each step, so
their rows are the queries of a step; the prefix rows' own attention, which yields the
prefix keys/values of the next layer, runs once per denoising step of a session ("3.3
Inference Acceleration and End-to-End Deployment", static-context KV caching: one bank per
denoising step).

  window_attention: moving row i (history chunks oldest first, then the current chunk)
    sees every key of the call's sequence -- the bank, the history and the whole current
    chunk.
  prefix_attention: prefix row i of a bank sees that bank's keys only.

Both are the masked-attention definition with an all-visible mask over the stated keys.
"""
import numpy as np

from .attention import masked_attention, widen


def window_attention(cache, bank, q, scale, dtype, heads=None, rows=None, row_block=2048):
    """q [M][H][D] storage array of the moving rows (M = history + current tokens)
    -> (o [len(rows)][len(heads)][D], lse [len(heads)][len(rows)]) fp64."""
    k, v, _ = cache.sequence(bank)
    n_moving = k.shape[0] - cache.prefix_len(bank)
    if q.shape[0] != n_moving:
        raise ValueError("queries are the moving rows: history then current tokens")
    return _dense(q, k, v, scale, dtype, heads, rows, row_block)


def prefix_attention(cache, bank, q, scale, dtype, heads=None, rows=None, row_block=2048):
    """q [P][H][D] storage array of bank `bank`'s prefix rows -> (o, lse) as above."""
    if not 0 <= bank < cache.banks:
        raise ValueError("bank out of range")
    if q.shape[0] != cache.prefix_len(bank) or q.shape[0] == 0:
        raise ValueError("queries are the prefix rows of the bank")
    return _dense(q, cache.pk[bank], cache.pv[bank], scale, dtype, heads, rows, row_block)


def _dense(q, k, v, scale, dtype, heads, rows, row_block):
    n_heads = q.shape[1]
    heads = list(range(n_heads)) if heads is None else list(heads)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    o = np.zeros((len(rows), len(heads), v.shape[2]))
    lse = np.zeros((len(heads), len(rows)))
    for hi, h in enumerate(heads):
        kh = widen(k[:, h, :], dtype)
        vh = widen(v[:, h, :], dtype)
        for r0 in range(0, len(rows), row_block):
            rb = rows[r0:r0 + row_block]
            ob, lb = masked_attention(widen(q[rb, h, :], dtype), kh, vh, np.ones((len(rb), kh.shape[0]), bool), scale)
            o[r0:r0 + len(rb), hi, :] = ob
            lse[hi, r0:r0 + len(rb)] = lb
    return o, lse
