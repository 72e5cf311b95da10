"""The plain C++ fp64 oracle against the pins, against the numpy oracle, and exhaustively on
tiny streams (CPU only).

The pins are the same callables-taking functions the numpy oracle is held to (tests/pins.py);
the cross-checks compare two implementations that share no code; the exhaustive enumeration
walks every order of appends, re-appends and evictions up to a fixed depth on tiny shapes and
checks each state against a direct evaluation of the window rule written here.
"""
import itertools
import math

import numpy as np
import pytest

import harness
import oracle
import pins
import synth
from oracle import native


@pytest.mark.parametrize("pin", pins.ALL_ATTENTION_PINS, ids=lambda f: f.__name__)
def test_native_attention_definition(pin):
    pin(native.masked_attention)


@pytest.mark.parametrize("window,cb", [(2, 3), (0, 7), (1, 1), (3, 2)])
def test_native_stream_equals_full_sequence(window, cb):
    """Streaming through the C++ cache == the C++ dense route == the numpy dense route."""
    for full in (native.full_sequence_attention, oracle.full_sequence_attention):
        pins.pin_stream_equals_full_sequence(native.StreamingCache, native.chunk_attention, full, window=window,
                                             causal_block=cb, n_chunks=7, seed=window * 10 + cb)


def test_native_stream_brute_force():
    pins.pin_stream_brute_force(native.StreamingCache, native.chunk_attention)


def test_native_window_rule():
    pins.pin_window_rule(native.StreamingCache)


def test_native_update_rule():
    pins.pin_update_rule(native.StreamingCache)


def _run_both(w, rows=None):
    """Streams workload w through both oracles; after every call compares the logical
    sequences bit for bit and the chunk attention within fp64 rounding."""
    stream = synth.SessionStream(w)
    pk, pv = stream.persistent()
    a = oracle.StreamingCache(pk, pv, w.window)
    b = native.StreamingCache(pk, pv, w.window)
    scale = 1.0 / math.sqrt(w.head_dim)
    worst = 0.0
    for st in stream:
        if st["evict_before"]:
            assert a.evict() == b.evict()
        a.append(st["chunk"], st["k"], st["v"])
        b.append(st["chunk"], st["k"], st["v"])
        assert a.visible_ids() == b.visible_ids()
        for bank in range(w.banks):
            ka, va, na = a.sequence(bank)
            kb, vb, nb = b.sequence(bank)
            assert na == nb and ka.dtype == kb.dtype and (ka == kb).all() and (va == vb).all()
        oa, la = oracle.chunk_attention(a, st["bank"], st["q"], scale, w.causal_block, w.dtype, rows=rows)
        ob, lb = native.chunk_attention(b, st["bank"], st["q"], scale, w.causal_block, w.dtype, rows=rows)
        assert np.abs(oa - ob).max() <= 1e-13 * max(1.0, np.abs(oa).max()), st["chunk"]
        assert np.abs(la - lb).max() <= 1e-12 * max(1.0, np.abs(la).max()), st["chunk"]
        worst = max(worst, float(np.abs(oa - ob).max()))
    return worst


@pytest.mark.parametrize("name", ["c0", "t_stream", "t_frame", "t_d64", "t_f32"])
def test_native_matches_numpy_streams(name):
    _run_both(synth.get_workload(name))


def test_native_matches_numpy_c1_sampled():
    """One chunk-step at c1's full size (4680 queries over 16112 keys, 24 heads) on sampled rows."""
    _run_both(synth.get_workload("c1"), rows=np.arange(0, 4680, 97))


def test_native_threads_do_not_change_results():
    w = synth.get_workload("t_frame")
    stream = synth.SessionStream(w)
    pk, pv = stream.persistent()
    c = native.StreamingCache(pk, pv, w.window)
    last = None
    for st in stream:
        if st["evict_before"]:
            c.evict()
        c.append(st["chunk"], st["k"], st["v"])
        last = st
    outs = [native.chunk_attention(c, 0, last["q"], 0.0884, w.causal_block, w.dtype, threads=t) for t in (1, 3, 0)]
    for o, l in outs[1:]:
        assert (o == outs[0][0]).all() and (l == outs[0][1]).all()


# ---------------------------------------------------------------- exhaustive tiny orders

def _direct(q, K, V, limit, scale):
    """Attention of one row over the first `limit` keys, straight from the formula (no max
    shift: the logits here are small), sums by math.fsum."""
    w = [math.exp(scale * math.fsum(float(a) * float(b) for a, b in zip(q, K[j]))) for j in range(limit)]
    l = math.fsum(w)
    o = [math.fsum(w[j] * float(V[j][d]) for j in range(limit)) / l for d in range(V.shape[1])]
    return o, math.log(l)


_OPS = ("evict", ("same", 3), ("next", 2), ("next", 4), ("same", 1))


def _enumerate(W, H, D, P, cb, depth, seed):
    """Every sequence of operations from _OPS up to `depth`: each applied to both oracles and to
    the library's host ring (sr_ring_*); a rejected operation must be rejected by all three and
    change nothing.  Every reachable state with a current chunk is checked against _direct."""
    sr = harness.lib_module()
    r = np.random.default_rng(seed)
    f32 = lambda *s: (r.standard_normal(s) * 0.7).astype(np.float32)
    pk, pv = f32(1, P, H, D), f32(1, P, H, D)
    pool = {}  # (depth, op) -> chunk tensors, fixed so that equal paths see equal data

    def tensors(n, key):
        if key not in pool:
            pool[key] = (f32(n, H, D), f32(n, H, D), f32(n, H, D))
        return pool[key]

    cfg = sr.config_for(H, 64, max(P, 0), 4, W, cb, 1, sr.SR_F32)
    states = 0
    for path in itertools.chain.from_iterable(itertools.product(_OPS, repeat=n) for n in range(1, depth + 1)):
        a = oracle.StreamingCache(pk, pv, W)
        b = native.StreamingCache(pk, pv, W)
        ring = sr.sr_ring_create(cfg)
        # the model written here: committed ids/data in the window, current id/data
        hist, cur = [], None
        try:
            for step, op in enumerate(path):
                if op == "evict":
                    ok = bool(hist)
                    outs = []
                    for m in (a, b):
                        try:
                            outs.append(m.evict())
                        except Exception:
                            outs.append(None)
                    try:
                        outs.append(sr.sr_ring_evict(ring))
                    except sr.SrError:
                        outs.append(None)
                    if ok:
                        assert outs == [hist[0][0]] * 3, (path, outs)
                        hist.pop(0)
                    else:
                        assert outs == [None] * 3, (path, outs)
                    continue
                kind, n = op
                cid = (0 if cur is None else cur[0]) + (1 if kind == "next" and cur is not None else 0)
                ok = cur is None or kind == "same" or W == 0 or len(hist) < W
                k, v, q = tensors(n, (step, op))
                res = []
                for m in (a, b):
                    try:
                        m.append(cid, k, v)
                        res.append(True)
                    except Exception:
                        res.append(False)
                try:
                    sr.sr_ring_append(ring, cid, n)
                    res.append(True)
                except sr.SrError:
                    res.append(False)
                assert res == [ok] * 3, (path, res)
                if not ok:
                    continue
                if cur is not None and kind == "next" and W > 0:
                    hist.append(cur)
                cur = (cid, k, v, q)
            if cur is None:
                continue
            # ids and the logical sequence
            ids = [h[0] for h in hist] + [cur[0]]
            assert a.visible_ids() == ids and b.visible_ids() == ids, path
            segs = sr.sr_ring_segments(ring, 0)  # (chunk_id, kind, slot, page, length)
            assert [g[0] for g in segs if g[1] != 0] == ids, path
            assert [g[4] for g in segs if g[1] != 0] == [h[1].shape[0] for h in hist] + [cur[1].shape[0]], path
            assert [g[4] for g in segs if g[1] == 0] == ([P] if P else []), path
            K = np.concatenate([pk[0]] + [h[1] for h in hist] + [cur[1]])
            V = np.concatenate([pv[0]] + [h[2] for h in hist] + [cur[2]])
            for m in (a, b):
                ks, vs, nf = m.sequence(0)
                assert (ks == K).all() and (vs == V).all() and nf == K.shape[0] - cur[1].shape[0], path
            q = cur[3]
            n_cur, n_fix = q.shape[0], K.shape[0] - q.shape[0]
            oa, la = oracle.chunk_attention(a, 0, q, 0.8, cb, "f32")
            ob, lb = native.chunk_attention(b, 0, q, 0.8, cb, "f32")
            for h in range(H):
                for i in range(n_cur):
                    lim = n_fix + min(n_cur, (i // cb + 1) * cb)
                    o, l = _direct(q[i, h], K[:, h], V[:, h], lim, 0.8)
                    for got_o, got_l in ((oa, la), (ob, lb)):
                        assert np.abs(got_o[i, h] - o).max() <= 1e-13 * max(1.0, max(map(abs, o))), (path, h, i)
                        assert abs(got_l[h, i] - l) <= 1e-13 * max(1.0, abs(l)), (path, h, i)
            states += 1
        finally:
            sr.sr_ring_destroy(ring)
    return states


@pytest.mark.parametrize("W,H,D,P,cb,depth", [(0, 1, 1, 0, 1, 5), (1, 2, 4, 3, 2, 5), (2, 2, 3, 1, 4, 5),
                                              (2, 1, 4, 2, 1, 5)])
def test_exhaustive_tiny_orders(W, H, D, P, cb, depth):
    """Every order of appends (first, same id, next id; ragged lengths 1-4), re-appends and
    evictions up to `depth` operations, at H <= 2, D <= 4, P <= 3, chunks of <= 4 tokens and
    W <= 2: both oracles and the host ring agree on what is accepted, the visible ids, the
    logical sequence, and the attention of every row of every reachable state."""
    states = _enumerate(W, H, D, P, cb, depth, seed=W * 100 + H * 10 + D)
    assert states > 100
