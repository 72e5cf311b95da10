"""Workload recipes: shapes, distributions and chunk processes of the streaming attention.

Shapes follow the resolutions and chunk sizes on the StreamRender-H3 pages (an
832x480 or 1280x720 frame downsampled 16x per side gives 52x30 = 1560 or
80x45 = 3600 tokens per latent frame; chunks of three or two latent frames), with
the sink/prefix of reference-image tokens plus 512 prompt tokens and a rolling
window of past chunks ("A window that slides, and a prefix that doesn't" on the
teardown page; "3.1.2 Historical Context and Temporal Consistency" on the
project page).  Head counts and head width are stand-ins: the pages do not give
H3's attention geometry.

Every tensor is drawn from a named counter-based sub-stream (see rng.py), as
fp32 (Gaussian * std) and, for bf16 workloads, rounded to bf16 bit patterns.
Layouts are token-major: chunk tensors [n][H][D], persistent banks [banks][P][H][D].
"""
from dataclasses import dataclass, replace
import math
import numpy as np

from .rng import substream_seed, uniform01
from ._native import normal_f64, f32_to_bf16

_SIGMA = 1.0 / math.sqrt(128.0)


@dataclass(frozen=True)
class Workload:
    name: str
    index: int            # seed offset: base seed = 20261012 + index
    dtype: str            # "bf16" or "f32" storage / input type
    heads: int
    head_dim: int
    persistent: int       # P: reference-image + prompt tokens per bank
    chunk: int            # tokens per chunk (= queries per attention call)
    window: int           # W: past chunks kept in the window
    causal_block: int     # tokens per causal block inside the current chunk
    banks: int            # persistent banks (one per denoising step)
    chunks: int           # chunks streamed in the session
    steps: int            # denoising steps per chunk
    qk_std: float
    v_std: float
    boost_fraction: float = 0.0   # fraction of visible key tokens scaled by `boost`
    boost: float = 30.0
    ar_rho: float = 0.0           # AR(1) coefficient of the chunk process (0: iid)
    single_step: bool = True      # only the last chunk-step (full window) is of interest

    @property
    def seed(self):
        return 20261012 + self.index

    @property
    def visible_keys(self):
        """Keys visible to the last block of the current chunk at full window."""
        return self.persistent + min(self.window, self.chunks - 1) * self.chunk + self.chunk

    def scaled(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    # tiny oracle check: fp32, 2 heads x 64, 16 persistent tokens, window 2 x 32, 4 chunks streamed
    "c0": Workload("c0", 0, "f32", 2, 64, 16, 32, 2, 32, 1, 4, 1, 1.0, 1.0, single_step=False),
    # 832x480 chunk-step: 24 heads, 1560 ref + 512 prompt, 2 past chunks of 3 frames x 1560
    "c1": Workload("c1", 1, "bf16", 24, 128, 2072, 4680, 2, 4680, 1, 3, 1, _SIGMA, _SIGMA),
    # streaming session at c1 shapes: 32 chunks x 2 steps, bank per step, AR(1) rho=0.9 chunk process
    "c2": Workload("c2", 2, "bf16", 24, 128, 2072, 4680, 2, 4680, 2, 32, 2, _SIGMA, _SIGMA,
                   ar_rho=0.9, single_step=False),
    # 720p chunk-step: 40 heads, 3600 ref + 512 prompt, 3 past chunks of 2 frames x 3600
    "c3": Workload("c3", 3, "bf16", 40, 128, 4112, 7200, 3, 7200, 1, 4, 1, _SIGMA, _SIGMA),
    # semantic-conditioned stress: frames of 1560 video + 1560 semantic tokens, frame-causal,
    # 32 heads, 1% of visible keys scaled x30
    "c4": Workload("c4", 4, "bf16", 32, 128, 2072, 9360, 2, 3120, 1, 3, 1, _SIGMA, _SIGMA,
                   boost_fraction=0.01),
    # stress variants: unit-variance Q,K so logits are O(1) (and O(100) on boosted keys)
    "c1s": Workload("c1s", 11, "bf16", 24, 128, 2072, 4680, 2, 4680, 1, 3, 1, 1.0, _SIGMA),
    "c4s": Workload("c4s", 14, "bf16", 32, 128, 2072, 9360, 2, 3120, 1, 3, 1, 1.0, _SIGMA,
                    boost_fraction=0.01),
    # page-literal window variant at c1 shapes: the 3 x 4680 moving rows (2 history chunks and
    # the current one) attend to the whole window, 2072 + 14040 keys
    "c1w": Workload("c1w", 31, "bf16", 24, 128, 2072, 4680, 2, 4680, 1, 3, 1, _SIGMA, _SIGMA),
    # fused append at c1 shapes: the chunk's qkv projection output is normalised, rotated and
    # written by one kernel before the chunk attention of the prepared queries
    "c1p": Workload("c1p", 35, "bf16", 24, 128, 2072, 4680, 2, 4680, 1, 3, 1, _SIGMA, _SIGMA),
    # reduced shapes the oracle finishes in seconds; they still span several tiles and ragged tails
    "t_stream": Workload("t_stream", 21, "bf16", 3, 128, 300, 600, 2, 600, 2, 5, 2, 1.0, 1.0,
                         ar_rho=0.9, single_step=False),
    "t_frame": Workload("t_frame", 22, "bf16", 2, 128, 200, 780, 2, 390, 1, 3, 1, 1.0, _SIGMA,
                        boost_fraction=0.01),
    "t_d64": Workload("t_d64", 23, "bf16", 3, 64, 130, 333, 1, 111, 1, 3, 1, 1.0, 1.0),
    "t_f32": Workload("t_f32", 24, "f32", 3, 64, 70, 300, 2, 100, 2, 5, 2, 1.0, 1.0, single_step=False),
    # window-variant streams: two banks, ragged tiles; fp32 and head_dim 64 too
    "t_win": Workload("t_win", 32, "bf16", 3, 128, 300, 420, 2, 420, 2, 5, 2, 1.0, 1.0, single_step=False),
    "t_win64": Workload("t_win64", 33, "bf16", 2, 64, 130, 200, 3, 200, 1, 5, 1, 1.0, 1.0, single_step=False),
    "t_winf32": Workload("t_winf32", 34, "f32", 2, 64, 70, 150, 1, 150, 2, 4, 2, 1.0, 1.0, single_step=False),
}


def get_workload(name):
    return WORKLOADS[name]


def _draw(w, tag, shape, std, chunk=0, step=0, bank=0):
    n = int(np.prod(shape))
    return normal_f64(substream_seed(w.seed, tag, chunk, step, bank), n, std).reshape(shape)


def _store(w, x64):
    """fp64 draw -> storage array (fp32, or bf16 bit patterns as uint16)."""
    f = np.asarray(x64, dtype=np.float32)
    return f32_to_bf16(f) if w.dtype == "bf16" else f


def _boost_positions(w):
    """Partial Fisher-Yates over the logical visible key sequence of the last chunk-step."""
    nk = w.visible_keys
    m = int(math.floor(w.boost_fraction * nk))
    if m == 0:
        return np.zeros(0, dtype=np.int64)
    u = uniform01(substream_seed(w.seed, "X30"), m)
    perm = np.arange(nk, dtype=np.int64)
    for i in range(m):
        j = i + int(math.floor(u[i] * (nk - i)))
        j = min(j, nk - 1)
        perm[i], perm[j] = perm[j], perm[i]
    return np.sort(perm[:m])


def persistent_inputs(w):
    """Persistent K/V banks, [banks][P][H][D] fp64 draws (before the boost and rounding)."""
    shape = (w.persistent, w.heads, w.head_dim)
    pk = np.stack([_draw(w, "PK", shape, w.qk_std, bank=b) for b in range(w.banks)]) if w.persistent else \
        np.zeros((w.banks, 0, w.heads, w.head_dim))
    pv = np.stack([_draw(w, "PV", shape, w.v_std, bank=b) for b in range(w.banks)]) if w.persistent else \
        np.zeros((w.banks, 0, w.heads, w.head_dim))
    return pk, pv


class SessionStream:
    """Seeded chunk-step stream of a workload.

    `persistent()` gives the stored persistent banks.  Iterating yields one dict per
    chunk-step in order: {"chunk", "step", "bank", "evict_before", "k", "v", "q"}.
    `evict_before` is True on the first step of a chunk that needs the oldest history
    chunk dropped (the window already holds W chunks).  For chunk processes with
    rho > 0 the last step of chunk c carries the committed K*_c, V*_c with
    K*_c = rho K*_{c-1} + sqrt(1 - rho^2) std eps_c; earlier steps carry
    rho K*_c + sqrt(1 - rho^2) std eta_c (a noisier version of the same chunk).
    """

    def __init__(self, w):
        self.w = w
        self._boost = _boost_positions(w) if w.boost_fraction > 0 else None

    def _boost_rows(self, x, start):
        """Scale the boosted logical key positions that fall in [start, start + len(x))."""
        if self._boost is None:
            return x
        sel = self._boost[(self._boost >= start) & (self._boost < start + x.shape[0])] - start
        if sel.size:
            x = x.copy()
            x[sel] *= self.w.boost
        return x

    def persistent(self):
        pk, pv = persistent_inputs(self.w)
        pk = np.stack([self._boost_rows(pk[b], 0) for b in range(self.w.banks)])
        return _store(self.w, pk), _store(self.w, pv)

    def __iter__(self):
        w = self.w
        shape = (w.chunk, w.heads, w.head_dim)
        kstar = vstar = None
        for c in range(w.chunks):
            if w.ar_rho > 0:
                a, b = w.ar_rho, math.sqrt(1.0 - w.ar_rho ** 2)
                ek = _draw(w, "KSTAR", shape, w.qk_std, chunk=c)
                ev = _draw(w, "VSTAR", shape, w.v_std, chunk=c)
                kstar = ek if kstar is None else a * kstar + b * ek
                vstar = ev if vstar is None else a * vstar + b * ev
            # before chunk c the window holds min(c - 1, W) committed chunks; it is full from c = W + 1 on
            evict = w.window > 0 and c >= w.window + 1
            # logical start of this chunk's keys in the last chunk-step's visible sequence (None: evicted)
            age = w.chunks - 1 - c
            start = w.persistent + (w.window - age) * w.chunk if (w.single_step and age <= w.window) else None
            for s in range(w.steps):
                if w.ar_rho > 0:
                    if s == w.steps - 1:
                        k, v = kstar, vstar
                    else:
                        k = a * kstar + b * _draw(w, "K_STEP0", shape, w.qk_std, chunk=c, step=s)
                        v = a * vstar + b * _draw(w, "V_STEP0", shape, w.v_std, chunk=c, step=s)
                else:
                    k = _draw(w, "K", shape, w.qk_std, chunk=c, step=s)
                    v = _draw(w, "V", shape, w.v_std, chunk=c, step=s)
                if start is not None:
                    k = self._boost_rows(k, start)
                q = _draw(w, "Q", shape, w.qk_std, chunk=c, step=s)
                yield {"chunk": c, "step": s, "bank": s % w.banks, "evict_before": evict and s == 0,
                       "k": _store(w, k), "v": _store(w, v), "q": _store(w, q)}


class WindowStream:
    """Seeded chunk-steps of the page-literal window variant of a workload.

    The moving part of the window (the history chunks still in it and the current chunk)
    is recomputed every step: each chunk-step draws fresh K/V for every history chunk in the
    window (tags KH/VH, keyed by the history chunk's id, the step and its distance to the
    current chunk), fresh K/V for the current chunk (K/V, as in SessionStream) and queries
    for every moving row (tag QM).  No boosted keys.  Every chunk has w.chunk tokens.
    `prefix_queries(bank)` draws the prefix rows' queries of a bank (tag QP).

    Yields per chunk-step {"chunk", "step", "bank", "evict_before", "history": [(id, k, v)]
    oldest first, "k", "v", "q"} with q the moving rows [M][H][D], history oldest first and
    then the current chunk's tokens.
    """

    def __init__(self, w):
        self.w = w

    def persistent(self):
        pk, pv = persistent_inputs(self.w)
        return _store(self.w, pk), _store(self.w, pv)

    def prefix_queries(self, bank):
        w = self.w
        return _store(w, _draw(w, "QP", (w.persistent, w.heads, w.head_dim), w.qk_std, bank=bank))

    def __iter__(self):
        w = self.w
        shape = (w.chunk, w.heads, w.head_dim)
        for c in range(w.chunks):
            evict = w.window > 0 and c >= w.window + 1
            ids = list(range(max(0, c - w.window), c))
            for s in range(w.steps):
                hist = [(i, _store(w, _draw(w, "KH", shape, w.qk_std, chunk=i, step=s, bank=c - i)),
                         _store(w, _draw(w, "VH", shape, w.v_std, chunk=i, step=s, bank=c - i))) for i in ids]
                k = _store(w, _draw(w, "K", shape, w.qk_std, chunk=c, step=s))
                v = _store(w, _draw(w, "V", shape, w.v_std, chunk=c, step=s))
                q = _store(w, _draw(w, "QM", ((len(ids) + 1) * w.chunk, w.heads, w.head_dim), w.qk_std, chunk=c,
                                    step=s))
                yield {"chunk": c, "step": s, "bank": s % w.banks, "evict_before": evict and s == 0,
                       "history": hist, "k": k, "v": v, "q": q}


def latent_positions(n_tokens, frame_tokens, grid_w, first_frame):
    """int32 [n][3] (t, y, x) of a chunk's tokens laid out frame by frame, row by row: token i
    is in latent frame first_frame + i // frame_tokens (stream-absolute), at grid row
    (i % frame_tokens) // grid_w and column i % grid_w."""
    i = np.arange(n_tokens)
    f = i % frame_tokens
    return np.stack([first_frame + i // frame_tokens, f // grid_w, f % grid_w], axis=1).astype(np.int32)


def qkv_inputs(w, n_tokens, chunk=0, step=0):
    """Seeded output of a qkv projection: storage array [n][3][H][D] (q and k ~ N(0, 1), v with
    the workload's v_std)."""
    shape = (n_tokens, 3, w.heads, w.head_dim)
    x = _draw(w, "QKV", shape, 1.0, chunk=chunk, step=step)
    x[:, 2] *= w.v_std
    return _store(w, x)


def prep_gains(w):
    """RMSNorm gains of q and k: fp32 [D] each, uniform-ish around 1 (drawn as 1 + 0.25 N(0,1))."""
    gq = 1.0 + _draw(w, "GQ", (w.head_dim,), 0.25)
    gk = 1.0 + _draw(w, "GK", (w.head_dim,), 0.25)
    return gq.astype(np.float32), gk.astype(np.float32)


def single_step_inputs(w):
    """Persistent banks, the W history chunks and the current chunk of a single-step workload.

    Returns (pk, pv, history [(k, v)] oldest first, (k, v, q) current)."""
    pk, pv = SessionStream(w).persistent()
    hist, cur = [], None
    for ev in SessionStream(w):
        if ev["chunk"] < w.chunks - 1:
            if ev["step"] == w.steps - 1:
                hist.append((ev["k"], ev["v"]))
        else:
            cur = (ev["k"], ev["v"], ev["q"])
    return pk, pv, hist[-w.window:] if w.window else [], cur


# ---------------------------------------------------------------- streaming decoder windows
# Project page, "3.2 Fast Causal H3 VAE": chunks of two latent frames, each attending to itself and
# the cached four before it, inside non-overlapping 16 x 16-token windows (every other layer
# shifted by half a window), plus five global (register and class) tokens rebuilt per chunk.  The
# latent grid of a 720p frame is 45 x 80 tokens (16x downsampling per side, as for the renderer's
# frames); head count and width are stand-ins (the pages give none for the decoder).

@dataclass(frozen=True)
class DecoderWorkload:
    name: str
    index: int            # seed offset: base seed = 20261012 + index
    heads: int
    head_dim: int
    grid_h: int           # latent tokens per frame: grid_h x grid_w
    grid_w: int
    window: int           # window side in tokens
    shift: int            # window offset (0, or half a window on shifted layers)
    frames: int           # latent frames per chunk
    window_chunks: int    # cached chunks (W)
    global_tokens: int
    chunks: int
    qk_std: float = 1.0
    v_std: float = 1.0
    dtype: str = "bf16"

    @property
    def seed(self):
        return 20261012 + self.index

    def partition(self):
        return window_partition(self.grid_h, self.grid_w, self.window, self.shift)

    @property
    def window_tokens(self):
        return [len(ix) for ix in self.partition()]

    @property
    def window_pages(self):
        return -(-self.frames * max(self.window_tokens) // 128)

    @property
    def chunk_tokens(self):
        return self.frames * self.grid_h * self.grid_w

    @property
    def capacity(self):
        """Slot capacity (tokens) of a cache holding every window's pages."""
        return len(self.window_tokens) * self.window_pages * 128

    def scaled(self, **kw):
        return replace(self, **kw)


def _cuts(n, window, shift):
    """Window boundaries along one axis: multiples of `window` moved back by `shift`."""
    inner = [k * window - shift for k in range(1, n // window + 2) if 0 < k * window - shift < n]
    return [0] + inner + [n]


def window_partition(grid_h, grid_w, window, shift):
    """Windows of one latent frame, row-major: a list of int arrays of the frame's token indices
    (row-major inside each window)."""
    rows, cols = _cuts(grid_h, window, shift), _cuts(grid_w, window, shift)
    out = []
    for r0, r1 in zip(rows[:-1], rows[1:]):
        for c0, c1 in zip(cols[:-1], cols[1:]):
            rr, cc = np.meshgrid(np.arange(r0, r1), np.arange(c0, c1), indexing="ij")
            out.append((rr * grid_w + cc).ravel())
    return out


def pack_windows(x, partition, frames, frame_tokens):
    """Frame-major chunk rows [frames * frame_tokens][...] -> packed window by window (window w:
    its tokens of frame 0, then frame 1, ...)."""
    order = np.concatenate([np.concatenate([f * frame_tokens + ix for f in range(frames)]) for ix in partition])
    return x[order]


DECODER_WORKLOADS = {
    # 720p decoder layer: 45 x 80 latent tokens per frame, 15 windows (10 of 16 x 16, 5 of 13 x 16)
    "d1": DecoderWorkload("d1", 41, 16, 128, 45, 80, 16, 0, 2, 2, 5, 4),
    # the shifted layer: 24 windows (edges of 8, 16, 16, 5 rows and 8, 16, 16, 16, 16, 8 columns)
    "d1s": DecoderWorkload("d1s", 42, 16, 128, 45, 80, 16, 8, 2, 2, 5, 4),
    # parity cases: several windows of two sizes, a shifted layout, a one-window multi-page layout
    "t_dec": DecoderWorkload("t_dec", 43, 3, 128, 20, 24, 8, 0, 2, 2, 5, 5),
    "t_dec_s": DecoderWorkload("t_dec_s", 44, 2, 128, 20, 24, 8, 4, 2, 2, 5, 5),
    "t_dec64": DecoderWorkload("t_dec64", 45, 2, 64, 16, 16, 16, 0, 2, 2, 5, 4),
    "t_decf32": DecoderWorkload("t_decf32", 46, 2, 64, 12, 12, 8, 0, 2, 1, 3, 4, dtype="f32"),
    # the most windows a layout takes (64), each one token per frame: every key tile nearly empty
    "t_decmax": DecoderWorkload("t_decmax", 47, 2, 128, 8, 8, 1, 0, 2, 2, 5, 4),
}


def get_decoder_workload(name):
    return DECODER_WORKLOADS[name]


class DecoderStream:
    """Seeded chunks of a decoder workload.  Yields per chunk {"chunk", "evict_before", "gk", "gv",
    "gq" [G][H][D] (the global tokens, rebuilt per chunk), "k", "v", "q" [T][H][D] packed window by
    window}.  Frame tokens are drawn frame-major (tags DK/DV/DQ) and packed with pack_windows."""

    def __init__(self, w):
        self.w = w

    def __iter__(self):
        w = self.w
        part = w.partition()
        ft = w.grid_h * w.grid_w
        shape = (w.frames * ft, w.heads, w.head_dim)
        gshape = (w.global_tokens, w.heads, w.head_dim)
        st = _store if w.dtype == "bf16" else (lambda _w, x: np.asarray(x, dtype=np.float32))
        for c in range(w.chunks):
            evict = w.window_chunks > 0 and c >= w.window_chunks + 1
            ev = {"chunk": c, "evict_before": evict}
            for tag, key, std in (("DGK", "gk", w.qk_std), ("DGV", "gv", w.v_std), ("DGQ", "gq", w.qk_std)):
                ev[key] = st(w, _draw(w, tag, gshape, std, chunk=c))
            for tag, key, std in (("DK", "k", w.qk_std), ("DV", "v", w.v_std), ("DQ", "q", w.qk_std)):
                ev[key] = st(w, pack_windows(_draw(w, tag, shape, std, chunk=c), part, w.frames, ft))
            yield ev
