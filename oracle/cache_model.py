"""The streaming KV cache as plain Python state (the oracle's own model).

Keys/values that a chunk-step attends to (project page "3.3 Inference
Acceleration and End-to-End Deployment", static-context KV caching: the static
context -- text/image conditioning, reference image, sink -- is computed once
per denoising timestep, each timestep keeps its own bank; the dynamic context of
recent and current frames moves with the stream; "3.2 Fast Causal H3 VAE": new
entries go into a preallocated ring and empty slots are hidden, never attended):

  * persistent[bank]: fixed for the session, one bank per denoising step;
  * history: the committed chunks still in the window, oldest first, at most W;
  * current: the chunk being denoised.  Appending the same id again replaces it
    (the next denoising step of the same chunk); appending id + 1 first commits
    the current chunk to the history (its last appended K/V is what stays).
  * evict drops the oldest history chunk.

Contract of the state machine (the HIP library follows the same rules; each
side implements them on its own):
  first append: any id >= 0; same id: overwrite; id == current + 1: commit then
  write -- an error if the history already holds W chunks (evict first; with
  W == 0 the committed chunk is simply dropped); any other id: error.
  evict with an empty history: error.  Errors leave the state unchanged.
Stored arrays are kept exactly as given (storage dtype), so the logical
sequence can be compared bit for bit with the device cache.
"""
from collections import deque

import numpy as np


class CacheStateError(Exception):
    """An append/evict that the state machine rejects (state unchanged)."""


class StreamingCache:
    def __init__(self, persistent_k, persistent_v, window, capacity=None):
        # persistent_k/v: [banks][P][H][D] storage arrays
        self.pk = [np.array(b) for b in persistent_k]
        self.pv = [np.array(b) for b in persistent_v]
        if len(self.pk) != len(self.pv) or not self.pk:
            raise ValueError("need >= 1 bank of persistent K and V")
        if window < 0:
            raise ValueError("window must be >= 0")
        self.window = window
        self.capacity = capacity
        self.history = deque()          # (chunk_id, k, v), oldest first
        self.current = None             # (chunk_id, k, v)

    @property
    def banks(self):
        return len(self.pk)

    def append(self, chunk_id, k, v):
        k, v = np.array(k), np.array(v)
        if chunk_id < 0 or k.shape != v.shape or k.shape[0] == 0:
            raise CacheStateError("bad chunk id or shape")
        if self.capacity is not None and k.shape[0] > self.capacity:
            raise CacheStateError("chunk larger than the slot capacity")
        if self.current is None:
            self.current = (chunk_id, k, v)
        elif chunk_id == self.current[0]:
            self.current = (chunk_id, k, v)
        elif chunk_id == self.current[0] + 1:
            if self.window == 0:
                self.current = (chunk_id, k, v)
            elif len(self.history) == self.window:
                raise CacheStateError("window full: evict first")
            else:
                self.history.append(self.current)
                self.current = (chunk_id, k, v)
        else:
            raise CacheStateError("chunk ids must repeat the current id or advance by one")

    def update(self, chunk_id, k, v):
        """Replace, in place, the K/V of a chunk in the window: a history chunk or the current one.

        Page-literal reading of the window (project page "3.1.2 Historical Context and
        Temporal Consistency", prefix cache): only the fixed prefix is cached; the recent
        history and the current chunk are recomputed every step, so the keys/values of a
        history chunk change while it stays in the window.  Same shape rules as append; an
        id outside the window is an error and changes nothing."""
        k, v = np.array(k), np.array(v)
        if k.shape != v.shape or k.shape[0] == 0:
            raise CacheStateError("bad chunk shape")
        if self.capacity is not None and k.shape[0] > self.capacity:
            raise CacheStateError("chunk larger than the slot capacity")
        if self.current is not None and chunk_id == self.current[0]:
            self.current = (chunk_id, k, v)
            return
        for i, (cid, _, _) in enumerate(self.history):
            if cid == chunk_id:
                self.history[i] = (cid, k, v)
                return
        raise CacheStateError("chunk %d is not in the window" % chunk_id)

    def set_bank(self, bank, k, v):
        """Replace the persistent tokens of `bank` in place, same shape.  The streaming decoder's
        global (register and class) tokens are rebuilt for every chunk and never cached (project
        page, "3.2 Fast Causal H3 VAE", iteration 4); its cache keeps them in the bank."""
        k, v = np.array(k), np.array(v)
        if not 0 <= bank < self.banks:
            raise CacheStateError("bank out of range")
        if k.shape != self.pk[bank].shape or v.shape != self.pv[bank].shape:
            raise CacheStateError("a bank keeps its shape")
        self.pk[bank], self.pv[bank] = k, v

    def prefix_len(self, bank):
        """Persistent (prefix) tokens of `bank`."""
        return self.pk[bank].shape[0]

    def evict(self):
        if not self.history:
            raise CacheStateError("nothing to evict")
        return self.history.popleft()[0]

    def visible_ids(self):
        """Chunk ids the current chunk attends to, in logical order (history..., current)."""
        return [c for c, _, _ in self.history] + ([self.current[0]] if self.current else [])

    def sequence(self, bank):
        """Logical key/value sequence for a call on `bank`, in storage dtype:
        returns (k [N][H][D], v [N][H][D], n_fixed) where the first n_fixed tokens are
        persistent + history (visible to every query) and the rest is the current chunk."""
        if self.current is None:
            raise CacheStateError("no current chunk")
        if not 0 <= bank < self.banks:
            raise CacheStateError("bank out of range")
        ks = [self.pk[bank]] + [k for _, k, _ in self.history] + [self.current[1]]
        vs = [self.pv[bank]] + [v for _, _, v in self.history] + [self.current[2]]
        n_fixed = sum(x.shape[0] for x in ks[:-1])
        return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0), n_fixed
