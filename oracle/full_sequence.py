"""Dense attention over the whole stream with an explicit mask -- an independent path.

The stream is laid out as one sequence [prefix; chunk 0; chunk 1; ...; chunk c]
with no cache at all.  The mask is written from the window rule itself
(teardown page "A window that slides, and a prefix that doesn't"; project page
"3.1.2 Historical Context and Temporal Consistency"): the fixed prefix attends
only to itself, and the rows of chunk c attend to the prefix, to the W chunks
immediately before c, and to the tokens of chunk c in causal blocks up to their
own.  The softmax goes through scipy's log-sum-exp, another rounding route than
the max-shift in attention.py, so agreement checks the cache bookkeeping
(which chunks are visible, in which order) and the arithmetic at once.
"""
import numpy as np
from scipy.special import logsumexp

from .attention import widen


def stream_mask(prefix_len, chunk_lens, window, causal_block, rows_of_chunk):
    """bool mask [n_rows, N] for the query rows `rows_of_chunk` (indices inside the last chunk)."""
    c = len(chunk_lens) - 1
    n = prefix_len + sum(chunk_lens)
    rows = np.asarray(rows_of_chunk)
    mask = np.zeros((len(rows), n), dtype=bool)
    mask[:, :prefix_len] = True
    off = prefix_len
    for t, ln in enumerate(chunk_lens):
        if t < c and c - t <= window:
            mask[:, off:off + ln] = True
        elif t == c:
            j = np.arange(ln)
            mask[:, off:off + ln] = (j[None, :] // causal_block) <= (rows[:, None] // causal_block)
        off += ln
    return mask


def prefix_self_attention(prefix_k, prefix_v, q_prefix, scale, dtype):
    """Rows of the fixed prefix attend only to the prefix (builds a bank); [P][H][D] -> o fp64."""
    P, H, _ = prefix_k.shape
    o = np.zeros(q_prefix.shape[:2] + (prefix_v.shape[2],))
    for h in range(H):
        s = scale * (widen(q_prefix[:, h, :], dtype) @ widen(prefix_k[:, h, :], dtype).T)
        p = np.exp(s - logsumexp(s, axis=1, keepdims=True))
        o[:, h, :] = p @ widen(prefix_v[:, h, :], dtype)
    return o


def full_sequence_attention(prefix_k, prefix_v, chunks_k, chunks_v, q, window, causal_block, scale, dtype):
    """Attention of the last chunk's queries q [n][H][D] over the whole stream.

    chunks_k/v: every chunk of the stream so far, oldest first, the last one current
    (the K/V each chunk ended up with).  Returns (o [n][H][D], lse [H][n]) fp64."""
    K = np.concatenate([prefix_k] + list(chunks_k), axis=0)
    V = np.concatenate([prefix_v] + list(chunks_v), axis=0)
    n = q.shape[0]
    mask = stream_mask(prefix_k.shape[0], [x.shape[0] for x in chunks_k], window, causal_block, np.arange(n))
    H = q.shape[1]
    o = np.zeros((n, H, V.shape[2]))
    lse = np.zeros((H, n))
    for h in range(H):
        s = scale * (widen(q[:, h, :], dtype) @ widen(K[:, h, :], dtype).T)
        s[~mask] = -np.inf
        lz = logsumexp(s, axis=1, keepdims=True)
        o[:, h, :] = np.exp(s - lz) @ widen(V[:, h, :], dtype)
        lse[h] = lz[:, 0]
    return o, lse


def window_mask(prefix_len, moving_len):
    """bool [P + M, P + M] over one window laid out as [prefix; moving part]: prefix rows
    see the prefix columns only, moving rows see every column (bidirectional window)."""
    n = prefix_len + moving_len
    mask = np.ones((n, n), dtype=bool)
    mask[:prefix_len, prefix_len:] = False
    return mask


def window_full_attention(prefix_k, prefix_v, moving_k, moving_v, q_prefix, q_moving, scale, dtype):
    """Every row of one window as a query over the window itself, with the asymmetric mask
    of the prefix cache (project page "3.1.2 Historical Context and Temporal Consistency").
    moving_k/v: the moving part's chunks oldest first (lists of [n][H][D]); q_prefix [P][H][D],
    q_moving [M][H][D].  Returns (o [P+M][H][D], lse [H][P+M]) fp64, prefix rows first."""
    K = np.concatenate([prefix_k] + list(moving_k), axis=0)
    V = np.concatenate([prefix_v] + list(moving_v), axis=0)
    Q = np.concatenate([q_prefix, q_moving], axis=0)
    mask = window_mask(prefix_k.shape[0], K.shape[0] - prefix_k.shape[0])
    H = Q.shape[1]
    o = np.zeros((Q.shape[0], H, V.shape[2]))
    lse = np.zeros((H, Q.shape[0]))
    for h in range(H):
        s = scale * (widen(Q[:, h, :], dtype) @ widen(K[:, h, :], dtype).T)
        s[~mask] = -np.inf
        lz = logsumexp(s, axis=1, keepdims=True)
        o[:, h, :] = np.exp(s - lz) @ widen(V[:, h, :], dtype)
        lse[h] = lz[:, 0]
    return o, lse
