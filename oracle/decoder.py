"""Window attention of the streaming causal decoder, in fp64.

What the step computes (project page, "3.2 Fast Causal H3 VAE"):
  * iteration 2 (time): the decoder works on chunks of two latent frames; every layer's
    attention of a chunk sees its own latent frames and the cached keys/values of the four
    before it, never a later one;
  * iteration 2 (space): attention runs inside non-overlapping windows of 16 x 16 tokens (every
    other layer shifts the windows by half a window), so a window's tokens attend to the same
    window's tokens only;
  * iteration 3, item 4: the attention of a window is computed as an independent sequence of
    its own (at 720p: 512 query rows, 1,541 keys), with no padded rows and with ring slots that
    hold nothing yet (the first chunks of a stream) left out of the key list;
  * iterations 4 and 6: four register tokens and one class token ("global tokens") attend to the
    whole frame, are rebuilt for every chunk and never cached; every window's attention also sees
    them (the 1,541 keys are 6 x 256 frame tokens + 5 global tokens).

Reading of the layout (listed with the design notes): a chunk's frame tokens arrive packed window by
window (window w: its tokens of the chunk's first latent frame, then of the second; n_w tokens per
latent frame, so frames x n_w per chunk).  The window attention of window w: its rows of the
current chunk over [global tokens | window w's tokens of the cached chunks, oldest first | window
w's tokens of the current chunk], all visible.  The global attention: the global tokens' queries
over [global tokens | every frame token of the current chunk], all visible (the cached frames are
other chunks' and the global tokens are rebuilt per chunk; reading: "the whole frame" is the
current chunk's).

The cache model is StreamingCache with one bank holding the chunk's global tokens (rewritten per
chunk with set_bank) and the packed frame tokens as chunks.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
import numpy as np

from .attention import masked_attention, widen


def window_offsets(window_tokens, frames):
    """Start of each window's rows in a packed chunk and the chunk's length."""
    sizes = frames * np.asarray(window_tokens, dtype=np.int64)
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    return starts, int(sizes.sum())


def window_rows(window_tokens, frames, w):
    """Row indices of window w in a packed chunk."""
    starts, _ = window_offsets(window_tokens, frames)
    return np.arange(starts[w], starts[w] + frames * int(window_tokens[w]))


def decoder_window_attention(cache, window_tokens, frames, q, scale, dtype, heads=None):
    """q [T][H][D] storage array: the current chunk's frame tokens, packed window by window.
    Returns (o [T][len(heads)][D], lse [len(heads)][T]) fp64: each window's rows over the global
    tokens (the bank), that window's rows of every history chunk (oldest first) and of the
    current chunk."""
    starts, total = window_offsets(window_tokens, frames)
    if q.shape[0] != total:
        raise ValueError("queries are the current chunk's packed frame tokens")
    gk, gv = cache.pk[0], cache.pv[0]
    chunks = [(k, v) for _, k, v in cache.history] + [(cache.current[1], cache.current[2])]
    for k, _ in chunks:
        if k.shape[0] != total:
            raise ValueError("every chunk has the same window layout")
    n_heads = q.shape[1]
    heads = list(range(n_heads)) if heads is None else list(heads)
    o = np.zeros((total, len(heads), q.shape[2]))
    lse = np.zeros((len(heads), total))
    for w in range(len(window_tokens)):
        rows = window_rows(window_tokens, frames, w)
        keys = np.concatenate([gk] + [k[rows] for k, _ in chunks], axis=0)
        vals = np.concatenate([gv] + [v[rows] for _, v in chunks], axis=0)
        for hi, h in enumerate(heads):
            ob, lb = masked_attention(widen(q[rows, h], dtype), widen(keys[:, h], dtype), widen(vals[:, h], dtype),
                                      np.ones((len(rows), keys.shape[0]), bool), scale)
            o[rows, hi] = ob
            lse[hi, rows] = lb
    return o, lse


def decoder_global_attention(cache, gq, scale, dtype, heads=None):
    """gq [G][H][D] storage array: the global tokens' queries.  Keys: the global tokens (the bank)
    and every frame token of the current chunk.  Returns (o [G][len(heads)][D], lse [len(heads)][G])."""
    gk, gv = cache.pk[0], cache.pv[0]
    ck, cv = cache.current[1], cache.current[2]
    keys = np.concatenate([gk, ck], axis=0)
    vals = np.concatenate([gv, cv], axis=0)
    n_heads = gq.shape[1]
    heads = list(range(n_heads)) if heads is None else list(heads)
    o = np.zeros((gq.shape[0], len(heads), gq.shape[2]))
    lse = np.zeros((len(heads), gq.shape[0]))
    for hi, h in enumerate(heads):
        o[:, hi], lse[hi] = masked_attention(widen(gq[:, h], dtype), widen(keys[:, h], dtype), widen(vals[:, h], dtype),
                                             np.ones((gq.shape[0], keys.shape[0]), bool), scale)
    return o, lse
