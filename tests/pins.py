"""Pins of the oracle against facts fixed by the pages and by the mathematics.

Each pin takes the oracle callables it checks as arguments, so that
test_oracle_mutations.py can run the same pins against copies of the oracle
with a planted mistake and show that the pin catches it.
"""
import math

import numpy as np

from oracle import brute_attention
from oracle.full_sequence import stream_mask


def _rng(seed):
    return np.random.default_rng(seed)


def pin_rows_sum_to_one(attn):
    """Every softmax row over the visible keys sums to 1 (hidden keys get 0)."""
    r = _rng(1)
    q, k, v = r.standard_normal((7, 5)), r.standard_normal((11, 5)), r.standard_normal((11, 3))
    vis = r.random((7, 11)) < 0.6
    vis[:, 0] = True
    _, _, p = attn(q, k, v, vis, 0.7, return_probs=True)
    assert np.abs(p.sum(axis=1) - 1.0).max() <= 1e-14
    assert (p[~vis] == 0).all()


def pin_single_key(attn):
    """One visible key: the output is that key's value, exactly; lse is its logit."""
    r = _rng(2)
    q, k, v = r.standard_normal((4, 6)), r.standard_normal((5, 6)), r.standard_normal((5, 6))
    vis = np.zeros((4, 5), dtype=bool)
    for i, j in enumerate([3, 0, 4, 3]):
        vis[i, j] = True
    o, lse = attn(q, k, v, vis, 0.3)
    for i, j in enumerate([3, 0, 4, 3]):
        assert (o[i] == v[j]).all()
        assert abs(lse[i] - 0.3 * float(q[i] @ k[j])) <= 1e-14 * max(1.0, abs(lse[i]))


def pin_equal_scores_mean(attn):
    """Equal logits (q = 0) give the mean of the visible values, and lse = ln(#visible)."""
    r = _rng(3)
    q = np.zeros((3, 4))
    k, v = r.standard_normal((9, 4)), r.standard_normal((9, 2))
    vis = np.ones((3, 9), dtype=bool)
    vis[1, 5:] = False
    vis[2, ::2] = False
    o, lse = attn(q, k, v, vis, 1.0)
    for i in range(3):
        m = v[vis[i]].mean(axis=0)
        assert np.abs(o[i] - m).max() <= 1e-15 * 10 * max(1.0, np.abs(m).max())
        assert abs(lse[i] - math.log(vis[i].sum())) <= 1e-14


def pin_two_key_closed_form(attn):
    """Logits {0, ln 3} give o = (v1 + 3 v2) / 4 and lse = ln 4 (scale != 1 on purpose)."""
    scale = 0.125
    q = np.array([[1.0, 0.0]])
    k = np.array([[0.0, 5.0], [math.log(3.0) / scale, -2.0]])
    v = np.array([[1.0, -2.0, 0.5], [3.0, 4.0, -1.5]])
    o, lse = attn(q, k, v, np.ones((1, 2), dtype=bool), scale)
    assert np.abs(o[0] - (v[0] + 3 * v[1]) / 4).max() <= 1e-15 * 4
    assert abs(lse[0] - math.log(4.0)) <= 1e-15 * 2


def pin_brute_force(attn, seeds=range(6)):
    """Random tiny problems against the decimal brute force (no max shift)."""
    for s in seeds:
        r = _rng(100 + s)
        nq, nk, d, dv = r.integers(1, 5), r.integers(1, 7), r.integers(1, 5), r.integers(1, 4)
        q, k, v = r.standard_normal((nq, d)) * 2, r.standard_normal((nk, d)) * 2, r.standard_normal((nk, dv))
        vis = r.random((nq, nk)) < 0.7
        vis[np.arange(nq), r.integers(0, nk, nq)] = True
        scale = float(r.uniform(0.1, 1.5))
        o, lse = attn(q, k, v, vis, scale)
        ob, lb = brute_attention(q.tolist(), k.tolist(), v.tolist(), vis.tolist(), scale)
        assert np.abs(o - np.array(ob)).max() <= 1e-13 * max(1.0, np.abs(ob).max())
        assert np.abs(lse - np.array(lb)).max() <= 1e-13 * max(1.0, np.abs(lb).max())


def pin_invariants(attn):
    """Shift of all keys by u, affine map of V, permutation of keys, convex hull."""
    r = _rng(4)
    q, k, v = r.standard_normal((6, 8)), r.standard_normal((13, 8)), r.standard_normal((13, 5))
    vis = r.random((6, 13)) < 0.5
    vis[:, 7] = True
    o, _ = attn(q, k, v, vis, 0.4)
    u = r.standard_normal(8)
    o2, _ = attn(q, k + u, v, vis, 0.4)          # adds 0.4*q.u to every logit of a row
    assert np.abs(o2 - o).max() <= 1e-12
    o3, _ = attn(q, k, 2.5 * v - 1.25, vis, 0.4)
    assert np.abs(o3 - (2.5 * o - 1.25)).max() <= 1e-12
    perm = r.permutation(13)
    o4, _ = attn(q, k[perm], v[perm], vis[:, perm], 0.4)
    assert np.abs(o4 - o).max() <= 1e-12
    for i in range(6):
        lo, hi = v[vis[i]].min(axis=0), v[vis[i]].max(axis=0)
        assert (o[i] >= lo - 1e-12).all() and (o[i] <= hi + 1e-12).all()


ALL_ATTENTION_PINS = [pin_rows_sum_to_one, pin_single_key, pin_equal_scores_mean, pin_two_key_closed_form,
                      pin_brute_force, pin_invariants]


# ---------------------------------------------------------------- streaming pins

def _tiny_stream(seed, n_chunks, steps, banks, P, Tc, H, D, dtype="f32"):
    r = _rng(seed)
    cast = (lambda a: a.astype(np.float32))
    pk = cast(r.standard_normal((banks, P, H, D)))
    pv = cast(r.standard_normal((banks, P, H, D)))
    chunks = []
    for c in range(n_chunks):
        chunks.append([(cast(r.standard_normal((Tc, H, D))), cast(r.standard_normal((Tc, H, D))),
                        cast(r.standard_normal((Tc, H, D)))) for _ in range(steps)])
    return pk, pv, chunks


def pin_stream_equals_full_sequence(cache_cls, chunk_attn, full_attn, window=2, causal_block=3, n_chunks=6,
                                    steps=2, banks=2, P=5, Tc=7, H=2, D=4, seed=7):
    """Chunk-by-chunk through the cache == one dense pass over the whole stream with the window mask."""
    pk, pv, chunks = _tiny_stream(seed, n_chunks, steps, banks, P, Tc, H, D)
    cache = cache_cls(pk, pv, window)
    committed_k, committed_v = [], []
    scale = 0.45
    for c in range(n_chunks):
        if window > 0 and c >= window + 1:
            cache.evict()
        for s in range(steps):
            k, v, q = chunks[c][s]
            cache.append(c, k, v)
            bank = s % banks
            o, lse = chunk_attn(cache, bank, q, scale, causal_block, "f32")
            of, lf = full_attn(pk[bank], pv[bank], committed_k + [k], committed_v + [v], q, window,
                               causal_block, scale, "f32")
            assert np.abs(o - of).max() <= 1e-12, (c, s)
            assert np.abs(lse - lf).max() <= 1e-12, (c, s)
        committed_k.append(chunks[c][steps - 1][0])
        committed_v.append(chunks[c][steps - 1][1])


def pin_stream_brute_force(cache_cls, chunk_attn, seeds=range(4)):
    """Tiny streams (all chunk-steps, evictions included) against the decimal brute force,
    the visible set written out from the window rule: prefix, last W committed chunks, own block."""
    for sd in seeds:
        r = _rng(200 + sd)
        W, cb, P, Tc, H, D = int(r.integers(0, 3)), int(r.integers(1, 5)), int(r.integers(1, 4)), \
            int(r.integers(1, 5)), int(r.integers(1, 3)), int(r.integers(1, 5))
        pk, pv, chunks = _tiny_stream(300 + sd, 4, 2, 1, P, Tc, H, D)
        cache = cache_cls(pk, pv, W)
        done = []
        for c in range(4):
            if W > 0 and c >= W + 1:
                cache.evict()
            for s in range(2):
                k, v, q = chunks[c][s]
                cache.append(c, k, v)
                o, _ = chunk_attn(cache, 0, q, 0.6, cb, "f32")
                hist = done[-W:] if W else []
                K = np.concatenate([pk[0]] + [x[0] for x in hist] + [k]).astype(np.float64)
                V = np.concatenate([pv[0]] + [x[1] for x in hist] + [v]).astype(np.float64)
                nfix = K.shape[0] - Tc
                for h in range(H):
                    vis = [[j < nfix or (j - nfix) // cb <= i // cb for j in range(K.shape[0])] for i in range(Tc)]
                    ob, _ = brute_attention(q[:, h].astype(np.float64).tolist(), K[:, h].tolist(), V[:, h].tolist(),
                                            vis, 0.6)
                    assert np.abs(o[:, h] - np.array(ob)).max() <= 1e-13 * max(1.0, np.abs(ob).max()), (sd, c, s, h)
            done.append(chunks[c][1])


def pin_window_rule(cache_cls, seed=11, n_ops=400):
    """After any valid sequence of appends/evicts, the visible chunk ids are the last
    (<= W) committed ids in order, then the current id; invalid calls change nothing."""
    r = _rng(seed)
    for W in range(0, 4):
        pk = np.zeros((1, 1, 1, 1), np.float32)
        cache = cache_cls(pk, pk, W)
        cur, hist = None, []
        x = np.zeros((1, 1, 1), np.float32)
        for _ in range(n_ops):
            op = r.integers(0, 4)
            if op == 0:
                try:
                    e = cache.evict()
                    assert hist and e == hist.pop(0)
                except Exception as ex:
                    assert not hist, ex
            else:
                cid = (int(r.integers(0, 1000)) if cur is None else
                       cur + (0 if op == 1 else 1 if op == 2 else int(r.integers(-3, 4))))
                ok = cid >= 0 and (cur is None or cid == cur or
                                   (cid == cur + 1 and (W == 0 or len(hist) < W)))
                try:
                    cache.append(cid, x, x)
                    assert ok
                    if cur is not None and cid == cur + 1 and W > 0:
                        hist.append(cur)
                    cur = cid
                except Exception as ex:
                    assert not ok, ex
            assert cache.visible_ids() == hist + ([cur] if cur is not None else [])


# ---------------------------------------------------------------- page-literal window pins

def _f32(r, *shape):
    return r.standard_normal(shape).astype(np.float32)


def pin_window_equals_full(cache_cls, window_attn, prefix_attn, full_attn, W=2, n_chunks=5, steps=2, banks=2,
                           P=5, Tc=4, H=2, D=3, seed=17):
    """A stream whose moving rows are recomputed every step (each history chunk updated in
    place, then the current chunk appended): the moving rows' attention through the cache,
    and the prefix rows' attention over their bank, equal one dense pass over the window
    [prefix; history; current] with the prefix cache's asymmetric mask."""
    r = _rng(seed)
    pk, pv = _f32(r, banks, P, H, D), _f32(r, banks, P, H, D)
    cache = cache_cls(pk, pv, W)
    scale = 0.55
    for c in range(n_chunks):
        if W > 0 and c >= W + 1:
            cache.evict()
        ids = [c - j for j in range(min(c, W), 0, -1)]
        for s in range(steps):
            kv = {cid: (_f32(r, Tc, H, D), _f32(r, Tc, H, D)) for cid in ids}
            for cid in ids:
                cache.update(cid, *kv[cid])
            kc, vc = _f32(r, Tc, H, D), _f32(r, Tc, H, D)
            cache.append(c, kc, vc)
            bank = s % banks
            qm, qp = _f32(r, Tc * (len(ids) + 1), H, D), _f32(r, P, H, D)
            o, lse = window_attn(cache, bank, qm, scale, "f32")
            op, lp = prefix_attn(cache, bank, qp, scale, "f32")
            of, lf = full_attn(pk[bank], pv[bank], [kv[i][0] for i in ids] + [kc], [kv[i][1] for i in ids] + [vc],
                               qp, qm, scale, "f32")
            assert np.abs(o - of[P:]).max() <= 1e-12 and np.abs(lse - lf[:, P:]).max() <= 1e-12, (c, s)
            assert np.abs(op - of[:P]).max() <= 1e-12 and np.abs(lp - lf[:, :P]).max() <= 1e-12, (c, s)


def pin_window_brute_force(cache_cls, window_attn, prefix_attn, seeds=range(3)):
    """Tiny windows against the decimal brute force, visible sets written out from the rule:
    a moving row sees prefix, history and current; a prefix row sees the prefix."""
    for sd in seeds:
        r = _rng(400 + sd)
        W, P, Tc, H, D = int(r.integers(1, 3)), int(r.integers(1, 4)), int(r.integers(1, 4)), 1, int(r.integers(1, 4))
        pk, pv = _f32(r, 1, P, H, D), _f32(r, 1, P, H, D)
        cache = cache_cls(pk, pv, W)
        ks, vs = [], []
        for c in range(W + 1):
            k, v = _f32(r, Tc, H, D), _f32(r, Tc, H, D)
            cache.append(c, k, v)
            ks.append(k)
            vs.append(v)
        K = np.concatenate([pk[0]] + ks).astype(np.float64)[:, 0]
        V = np.concatenate([pv[0]] + vs).astype(np.float64)[:, 0]
        qm, qp = _f32(r, Tc * (W + 1), H, D), _f32(r, P, H, D)
        o, lse = window_attn(cache, 0, qm, 0.8, "f32")
        ob, lb = brute_attention(qm[:, 0].astype(np.float64).tolist(), K.tolist(), V.tolist(),
                                 [[True] * K.shape[0]] * qm.shape[0], 0.8)
        assert np.abs(o[:, 0] - np.array(ob)).max() <= 1e-13 * max(1.0, np.abs(ob).max()), sd
        assert np.abs(lse[0] - np.array(lb)).max() <= 1e-13 * max(1.0, np.abs(lb).max()), sd
        op, _ = prefix_attn(cache, 0, qp, 0.8, "f32")
        ob, _ = brute_attention(qp[:, 0].astype(np.float64).tolist(), K[:P].tolist(), V[:P].tolist(),
                                [[True] * P] * P, 0.8)
        assert np.abs(op[:, 0] - np.array(ob)).max() <= 1e-13 * max(1.0, np.abs(ob).max()), sd


def pin_window_chunking_free(cache_cls, window_attn, seed=23):
    """Attention inside the window is bidirectional: the moving rows' results depend on the
    moving tokens only, not on how they are cut into chunks (here 9 tokens as 3 + 2 + 4 in a
    W = 2 window, and as 5 + 4 in a W = 1 window)."""
    r = _rng(seed)
    P, H, D = 3, 2, 4
    pk, pv = _f32(r, 1, P, H, D), _f32(r, 1, P, H, D)
    k, v, q = _f32(r, 9, H, D), _f32(r, 9, H, D), _f32(r, 9, H, D)
    a = cache_cls(pk, pv, 2)
    for cid, (lo, hi) in enumerate([(0, 3), (3, 5), (5, 9)]):
        a.append(cid, k[lo:hi], v[lo:hi])
    b = cache_cls(pk, pv, 1)
    for cid, (lo, hi) in enumerate([(0, 5), (5, 9)]):
        b.append(cid, k[lo:hi], v[lo:hi])
    oa, la = window_attn(a, 0, q, 0.5, "f32")
    ob, lb = window_attn(b, 0, q, 0.5, "f32")
    assert np.abs(oa - ob).max() <= 1e-13 and np.abs(la - lb).max() <= 1e-13


def pin_update_rule(cache_cls, seed=29):
    """update replaces exactly the named chunk of the window (history or current) and
    nothing else; an id outside the window is rejected with the state unchanged."""
    r = _rng(seed)
    pk = _f32(r, 1, 2, 1, 2)
    cache = cache_cls(pk, pk, 2)
    chunks = [(_f32(r, 3, 1, 2), _f32(r, 3, 1, 2)) for _ in range(3)]
    for cid, (k, v) in enumerate(chunks):
        cache.append(cid, k, v)
    k_new, v_new = _f32(r, 2, 1, 2), _f32(r, 2, 1, 2)
    cache.update(1, k_new, v_new)
    ks, vs, _ = cache.sequence(0)
    want_k = np.concatenate([pk[0], chunks[0][0], k_new, chunks[2][0]])
    want_v = np.concatenate([pk[0], chunks[0][1], v_new, chunks[2][1]])
    assert ks.shape == want_k.shape and (ks == want_k).all() and (vs == want_v).all()
    before = cache.sequence(0)
    for bad in (3, 7, -1):
        try:
            cache.update(bad, k_new, v_new)
            raise AssertionError("update of a chunk outside the window was accepted")
        except AssertionError:
            raise
        except Exception:
            pass
    after = cache.sequence(0)
    assert all((x == y).all() for x, y in zip(before[:2], after[:2])) and before[2] == after[2]
    cache.evict()
    try:
        cache.update(0, k_new, v_new)
        raise AssertionError("update of an evicted chunk was accepted")
    except AssertionError:
        raise
    except Exception:
        pass


# ---------------------------------------------------------------- qk-RMSNorm + rotary embedding pins

def pin_rms_norm(rms_norm):
    """Unit RMS with gamma = 1 and eps = 0; scale invariance; the eps closed form on a constant
    vector; gamma multiplies feature by feature."""
    r = _rng(51)
    x = r.standard_normal((5, 3, 16)) * 3.0
    y = rms_norm(x, np.ones(16), 0.0)
    assert np.abs(np.mean(y * y, axis=-1) - 1.0).max() <= 1e-14
    assert np.abs(rms_norm(7.5 * x, np.ones(16), 0.0) - y).max() <= 1e-14
    a, eps = 0.3, 0.05
    c = rms_norm(np.full((1, 8), a), np.ones(8), eps)
    assert np.abs(c - a / math.sqrt(a * a + eps)).max() <= 1e-15
    g = r.uniform(0.5, 2.0, 16)
    assert np.abs(rms_norm(x, g, 1e-6) - rms_norm(x, np.ones(16), 1e-6) * g).max() <= 1e-13


def pin_rope_closed_form(rope):
    """A unit vector on the first element of pair j turns by pos_a * base^(-k / n_a) into the
    pair (cos, sin); written out for one pair in each section, with base and sections chosen
    so the exponent and the section bookkeeping matter."""
    sections, base, D = (2, 3, 3), 500.0, 16
    cases = [(0, 0, 0), (1, 0, 1), (2, 1, 0), (4, 1, 2), (5, 2, 0), (7, 2, 2)]   # (pair j, axis a, index k)
    pos = np.array([[37, -5, 11]])
    for j, a, k in cases:
        x = np.zeros((1, 1, D))
        x[0, 0, 2 * j] = 1.0
        y = rope(x, pos, sections, base)
        ang = pos[0, a] * base ** (-k / sections[a])
        want = np.zeros(D)
        want[2 * j], want[2 * j + 1] = math.cos(ang), math.sin(ang)
        assert np.abs(y[0, 0] - want).max() <= 1e-12, (j, a, k)


def pin_rope_relative(rope, seed=53):
    """Scores depend only on position differences (project page 3.2, iteration 4): shifting
    both positions by the same amount on any axis leaves q'.k' unchanged; position 0 is the
    identity; pair norms are preserved; rotations compose."""
    r = _rng(seed)
    sections, base, D = (3, 2, 3), 10000.0, 16
    q, k = r.standard_normal((4, 2, D)), r.standard_normal((4, 2, D))
    pq = r.integers(-50, 50, (4, 3))
    pk = r.integers(-50, 50, (4, 3))
    s0 = np.einsum("nhd,nhd->nh", rope(q, pq, sections, base), rope(k, pk, sections, base))
    for shift in ([100, 0, 0], [0, -7, 0], [3, 5, 1000]):
        s1 = np.einsum("nhd,nhd->nh", rope(q, pq + shift, sections, base), rope(k, pk + shift, sections, base))
        assert np.abs(s1 - s0).max() <= 1e-9, shift
    assert np.abs(rope(q, np.zeros((4, 3), int), sections, base) - q).max() == 0.0
    y = rope(q, pq, sections, base)
    assert np.abs((y[..., 0::2] ** 2 + y[..., 1::2] ** 2) - (q[..., 0::2] ** 2 + q[..., 1::2] ** 2)).max() <= 1e-12
    p2 = r.integers(-50, 50, (4, 3))
    assert np.abs(rope(rope(q, pq, sections, base), p2, sections, base) - rope(q, pq + p2, sections, base)).max() <= 1e-11


def pin_rope_sections(rope, seed=57):
    """A pair only sees its own axis: changing the y position leaves the t and x pairs as they
    were, and so on for each axis."""
    r = _rng(seed)
    sections, base, D = (2, 3, 3), 10000.0, 16
    x = r.standard_normal((3, 1, D))
    pos = r.integers(0, 40, (3, 3))
    y0 = rope(x, pos, sections, base)
    bounds = np.cumsum((0,) + sections)
    for a in range(3):
        p = pos.copy()
        p[:, a] += 13
        y1 = rope(x, p, sections, base)
        own = np.zeros(D, bool)
        own[2 * bounds[a]:2 * bounds[a + 1]] = True
        assert (y1[..., ~own] == y0[..., ~own]).all(), a
        assert not np.allclose(y1[..., own], y0[..., own]), a


def pin_prep_qkv(prep_qkv, rms_norm, rope, seed=59):
    """q and k are normalised with their own gains and then rotated; v passes unchanged."""
    r = _rng(seed)
    n, H, D = 6, 2, 8
    qkv = r.standard_normal((n, 3, H, D)).astype(np.float32)
    pos = r.integers(0, 9, (n, 3))
    gq, gk = r.uniform(0.5, 2, D), r.uniform(0.5, 2, D)
    q, k, v = prep_qkv(qkv, pos, gq, gk, 1e-5, (2, 1, 1), 100.0, "f32")
    assert (v == qkv[:, 2].astype(np.float64)).all()
    # independent route: rotate a normalised vector pair by pair with explicit cos/sin
    for name, got, src, g in (("q", q, qkv[:, 0], gq), ("k", k, qkv[:, 1], gk)):
        xs = src.astype(np.float64)
        xn = xs / np.sqrt((xs ** 2).mean(-1, keepdims=True) + 1e-5) * g
        want = np.empty_like(xn)
        for i in range(n):
            for j in range(D // 2):
                a, kk, na = (0, j, 2) if j < 2 else ((1, 0, 1) if j == 2 else (2, 0, 1))
                ang = pos[i, a] * 100.0 ** (-kk / na)
                c, s = math.cos(ang), math.sin(ang)
                want[i, :, 2 * j] = xn[i, :, 2 * j] * c - xn[i, :, 2 * j + 1] * s
                want[i, :, 2 * j + 1] = xn[i, :, 2 * j] * s + xn[i, :, 2 * j + 1] * c
        assert np.abs(got - want).max() <= 1e-12, name
