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


# ---------------------------------------------------------------- MXFP6 / FP8 quantization pins
# The formats are those of the OCP Microscaling (MX) specification v1.0: the value sets
# below are the ones it publishes; the rounding rule is the nearest value, ties to the
# even mantissa, with saturation.  Each pin takes the oracle.mx module (or a copy with a
# planted mistake) as `m`.

# Magnitudes of FP6 E2M3 codes 0..31 as the specification lists them: 8 subnormals in
# steps of 1/8, then binades [1, 2), [2, 4), [4, 8) of 8 values each; largest 7.5.
E2M3_MAGNITUDES = [0.0, 0.125, 0.25, 0.375, 0.5, 0.625, 0.75, 0.875,
                   1.0, 1.125, 1.25, 1.375, 1.5, 1.625, 1.75, 1.875,
                   2.0, 2.25, 2.5, 2.75, 3.0, 3.25, 3.5, 3.75,
                   4.0, 4.5, 5.0, 5.5, 6.0, 6.5, 7.0, 7.5]


def pin_e2m3_values(m):
    """All 64 FP6 E2M3 codes decode to the published value set (sign bit 5 on top)."""
    for c in range(32):
        pos, neg = m.element_value(c, m.E2M3), m.element_value(32 + c, m.E2M3)
        assert pos == E2M3_MAGNITUDES[c] and not math.copysign(1.0, pos) < 0, c
        assert neg == -E2M3_MAGNITUDES[c] and math.copysign(1.0, neg) < 0, c


def pin_e4m3_values(m):
    """All 256 FP8 E4M3 codes decode as torch's float8_e4m3fn does (NaN at S.1111.111)."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([m.element_value(c, m.E4M3) for c in range(256)])
    assert (np.isnan(got) == np.isnan(ref)).all()
    ok = ~np.isnan(ref)
    assert (got[ok] == ref[ok]).all() and (np.signbit(got[ok]) == np.signbit(ref[ok])).all()
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9


def _nearest_codes(m, fmt, x):
    """Brute force: the code whose value is nearest to x, ties to the even code (the
    mantissa's last bit), magnitudes past the largest value saturating, sign from x."""
    width = 1 + fmt[0] + fmt[1]
    half = 1 << (width - 1)
    mags = np.array([m.element_value(c, fmt) for c in range(half)])
    ok = ~np.isnan(mags)
    idx = np.arange(half)[ok]
    mags = mags[ok]
    a = np.abs(x)[:, None]
    d = np.abs(a - mags[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates prefer the even code
    pick = np.where(cand & (idx[None, :] % 2 == 0), idx[None, :], -1).max(axis=1)
    single = cand.sum(axis=1) == 1
    pick = np.where(single, idx[np.argmax(cand, axis=1)], pick)
    return (pick | np.where(np.signbit(x), half, 0)).astype(np.int64)


def _encode_samples(m, fmt, r):
    width = 1 + fmt[0] + fmt[1]
    mags = np.array([m.element_value(c, fmt) for c in range(1 << (width - 1))])
    mags = np.sort(mags[~np.isnan(mags)])
    mids = (mags[1:] + mags[:-1]) / 2                      # exact ties
    tiny, big = mags[1], mags[-1]
    logu = np.exp2(r.uniform(np.log2(tiny) - 3, np.log2(big) + 2, 3000))
    x = np.concatenate([mags, mids, logu, mids * (1 + 1e-12), mids * (1 - 1e-12), [0.0, big * 1.06, big * 1e6]])
    sign = np.where(r.random(x.size) < 0.5, -1.0, 1.0)
    return np.concatenate([x * sign, [-0.0]])


def pin_encode_nearest(m, seed=61):
    """encode() picks the nearest value, ties to even, saturating, sign kept -- checked by
    brute force over every code of both formats, on exact ties and random magnitudes."""
    r = _rng(seed)
    for fmt in (m.E2M3, m.E4M3):
        x = _encode_samples(m, fmt, r)
        got = m.encode(x, fmt).astype(np.int64)
        want = _nearest_codes(m, fmt, x)
        assert (got == want).all(), (fmt, x[got != want][:5], got[got != want][:5], want[got != want][:5])


def pin_e4m3_encode_torch(m, seed=67):
    """Within +-448, FP8 E4M3 rounding agrees with torch's float32 -> float8_e4m3fn conversion
    (nearest, ties to even), bit for bit, including subnormals and signed zeros."""
    import torch
    r = _rng(seed)
    x = np.concatenate([r.standard_normal(4000) * np.exp2(r.integers(-12, 9, 4000)),
                        r.uniform(-448, 448, 1000), [0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -10, 447.9, -448.0]])
    x = x.astype(np.float32)
    x = np.clip(x, -448, 448).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = m.encode(x, m.E4M3)
    assert (got == ref).all(), (x[got != ref][:5], got[got != ref][:5], ref[got != ref][:5])
    assert (m.fp8_values(np.array([1000.0, -1e6, 460.0])) == [448.0, -448.0, 448.0]).all()


def pin_mx_scale(m, seed=71):
    """E8M0 block exponent: max |x| / 2^X lies in [4, 8) (E2M3's top binade), one exponent per
    32 consecutive elements, clamped at -127 (also for an all-zero block)."""
    r = _rng(seed)
    n, D = 200, 128
    x = r.standard_normal((n, D)) * np.exp2(r.integers(-100, 100, (n, 1)))
    x[0, :32] = 0.0
    x[1, :32] = r.uniform(-1, 1, 32) * 2.0 ** -140   # below the clamp
    x[2:4, :32] = r.uniform(-1, 1, (2, 32)) * 2.0 ** 39
    x[2, 5] = 2.0 ** 40                              # exact power of two as the block max
    x[3, 7] = 2.0 ** 40 * (1 - 2.0 ** -30)           # just below a power of two
    X = m.mx_scale_exponents(x)
    assert X.shape == (n, D // 32)
    amax = np.abs(x.reshape(n, D // 32, 32)).max(-1)
    ok = amax > 2.0 ** -120
    ratio = amax[ok] / np.exp2(X[ok])
    assert (ratio >= 4).all() and (ratio < 8).all()
    assert X[0, 0] == -127 and X[1, 0] == -127 and X[2, 0] == 38 and X[3, 0] == 37
    # one element changes only its own block's exponent, and elements 31 / 32 belong to
    # different blocks
    y = x[10:11].copy()
    y[0, 31] = 2.0 ** 60
    Xy = m.mx_scale_exponents(y)
    assert Xy[0, 0] == 58 and (Xy[0, 1:] == X[10, 1:]).all()
    y = x[10:11].copy()
    y[0, 32] = 2.0 ** 60
    Xy = m.mx_scale_exponents(y)
    assert Xy[0, 1] == 58 and Xy[0, 0] == X[10, 0] and (Xy[0, 2:] == X[10, 2:]).all()


def pin_mx_quantize(m, seed=73):
    """MXFP6 quantization: the textbook error bound of rounding to 3 mantissa bits (2^-4
    relative on the normal range, 2^(X-4) absolute below it, saturation at 7.5 2^X); values
    already on the grid come back unchanged; and a worked example by hand."""
    r = _rng(seed)
    n, D = 300, 64
    x = r.standard_normal((n, D)) * np.exp2(r.integers(-30, 30, (n, 1))) * r.uniform(0.01, 3, (n, D))
    codes, X = m.mx_quantize(x)
    assert codes.shape == x.shape and X.shape == (n, D // 32)
    deq = m.mx_dequantize(codes, X)
    Xe = np.repeat(X, 32, axis=1).astype(np.float64)
    u = np.abs(x) / np.exp2(Xe)
    err = np.abs(deq - x)
    sat = u > 7.5
    assert (deq[sat] == np.sign(x[sat]) * 7.5 * np.exp2(Xe[sat])).all()
    norm = (u >= 1) & ~sat
    assert (err[norm] <= 2.0 ** -4 * np.abs(x[norm])).all()
    assert (err[u < 1] <= np.exp2(Xe[u < 1] - 4)).all()
    assert (m.mxfp6_values(x) == deq).all()
    # grid values round-trip: random codes with one element of each block in [4, 7.5]
    c = r.integers(0, 64, (50, D)).astype(np.uint8)
    c[:, ::32] = (r.integers(24, 32, (50, D // 32)) | (r.integers(0, 2, (50, D // 32)) << 5)).astype(np.uint8)
    Xg = r.integers(-120, 120, (50, D // 32))
    g = m.mx_dequantize(c, Xg)
    c2, X2 = m.mx_quantize(g)
    assert (X2 == Xg).all() and (c2 == c).all()
    # by hand: block max 8 -> X = 3 - 2 = 1; 0.3 / 2 = 0.15 -> 0.125, -0.2 / 2 = -0.1 -> -0.125,
    # 15.6 / 2 would be 7.8 but the max is 8 here; 7.7 / 2 = 3.85 -> 3.75 (step 0.25)
    blk = np.zeros(32)
    blk[:5] = [8.0, 1.0, 0.3, -0.2, 7.7]
    assert (m.mxfp6_values(blk[None])[0, :5] == [8.0, 1.0, 0.25, -0.25, 7.5]).all()
    blk[0] = 15.5                                       # X = 1; 15.5 / 2 = 7.75 -> saturates to 7.5
    assert m.mxfp6_values(blk[None])[0, 0] == 15.0


# ---------------------------------------------------------------- streaming decoder window attention

def _decoder_stream(cache_cls, seed, window_tokens, frames, W, G, H, D, n_chunks, perturb=None):
    """A seeded decoder stream: per chunk, fresh global tokens (set_bank) and the packed frame tokens;
    returns the cache after the last chunk, that chunk's queries, the global queries, and every
    chunk's (k, v) (for the dense route).  perturb(c, k, v) may modify chunk c's arrays."""
    r = _rng(seed)
    T = frames * int(np.sum(window_tokens))
    f = lambda *s: r.standard_normal(s).astype(np.float32)
    cache = cache_cls(f(1, G, H, D), f(1, G, H, D), W)
    chunks = []
    for c in range(n_chunks):
        gk, gv = f(G, H, D), f(G, H, D)
        k, v = f(T, H, D), f(T, H, D)
        if perturb:
            k, v = perturb(c, k, v)
        cache.set_bank(0, gk, gv)
        if W and c > W:
            cache.evict()
        cache.append(c, k, v)
        chunks.append((k, v))
    return cache, f(T, H, D), f(G, H, D), chunks, (gk, gv)


def _decoder_dense(window_tokens, frames, W, chunks, glob, q, gq, scale):
    """Independent route: one masked attention per head over [global | every chunk still visible
    (the last W + 1), in stream order], with an explicit mask built from each key's chunk and
    window and each query's window."""
    gk, gv = glob
    vis_chunks = chunks[-(W + 1):]
    wid = np.repeat(np.arange(len(window_tokens)), frames * np.asarray(window_tokens))
    G = gk.shape[0]
    keys = np.concatenate([gk] + [k for k, _ in vis_chunks], axis=0).astype(np.float64)
    vals = np.concatenate([gv] + [v for _, v in vis_chunks], axis=0).astype(np.float64)
    key_w = np.concatenate([np.full(G, -1)] + [wid for _ in vis_chunks])
    key_c = np.concatenate([np.full(G, -1)] + [np.full(len(wid), i) for i in range(len(vis_chunks))])
    cur = len(vis_chunks) - 1
    qs = np.concatenate([q, gq], axis=0).astype(np.float64)
    mask = np.zeros((qs.shape[0], keys.shape[0]), bool)
    T = len(wid)
    mask[:T] = (key_w[None, :] == wid[:, None]) | (key_w[None, :] == -1)
    mask[T:] = (key_c[None, :] == cur) | (key_c[None, :] == -1)
    H = q.shape[1]
    o = np.zeros((qs.shape[0], H, q.shape[2]))
    lse = np.zeros((H, qs.shape[0]))
    from oracle import masked_attention
    for h in range(H):
        o[:, h], lse[h] = masked_attention(qs[:, h], keys[:, h], vals[:, h], mask, scale)
    return o[:T], lse[:, :T], o[T:], lse[:, T:]


def pin_decoder_equals_dense(cache_cls, win_attn, glob_attn):
    """The per-window routine and the global routine equal one dense masked attention over the
    visible stream, from the first chunk (no history: empty slots hidden) to a full, evicting
    window, on a ragged layout."""
    window_tokens, frames, W, G, H, D = [3, 2, 4, 1], 2, 2, 2, 2, 8
    for n_chunks in (1, 2, 3, 5):
        cache, q, gq, chunks, glob = _decoder_stream(cache_cls, 61 + n_chunks, window_tokens, frames, W, G, H, D,
                                                     n_chunks)
        o, lse = win_attn(cache, window_tokens, frames, q, 0.4, "f32")
        og, lg = glob_attn(cache, gq, 0.4, "f32")
        ro, rl, rog, rlg = _decoder_dense(window_tokens, frames, W, chunks, glob, q, gq, 0.4)
        assert np.abs(o - ro).max() <= 1e-12 and np.abs(lse - rl).max() <= 1e-12, n_chunks
        assert np.abs(og - rog).max() <= 1e-12 and np.abs(lg - rlg).max() <= 1e-12, n_chunks


def pin_decoder_brute(cache_cls, win_attn, glob_attn):
    """Decimal brute force on a tiny stream (two windows, W = 1, three chunks)."""
    from oracle import brute_attention
    window_tokens, frames, W, G, H, D = [1, 2], 2, 1, 1, 1, 3
    cache, q, gq, chunks, glob = _decoder_stream(cache_cls, 71, window_tokens, frames, W, G, H, D, 3)
    o, lse = win_attn(cache, window_tokens, frames, q, 0.7, "f32")
    og, lg = glob_attn(cache, gq, 0.7, "f32")
    ro, rl, rog, rlg = _decoder_dense(window_tokens, frames, W, chunks, glob, q, gq, 0.7)
    gk, gv = glob
    keys = np.concatenate([gk] + [k for k, _ in chunks[-2:]])[:, 0]
    vals = np.concatenate([gv] + [v for _, v in chunks[-2:]])[:, 0]
    wid = np.repeat([0, 1], [2, 4])
    kw = np.concatenate([[-1], wid, wid])
    vis = [[kw[j] in (-1, wid[i]) for j in range(len(kw))] for i in range(6)]
    bo, bl = brute_attention(q[:, 0].tolist(), keys.tolist(), vals.tolist(), vis, 0.7)
    assert np.abs(o[:, 0] - np.array(bo)).max() <= 1e-13 and np.abs(lse[0] - np.array(bl)).max() <= 1e-13
    kc = np.concatenate([[1], np.zeros(6), np.ones(6)])
    visg = [[bool(kc[j]) for j in range(len(kc))]]
    bog, blg = brute_attention(gq[:, 0].tolist(), keys.tolist(), vals.tolist(), visg, 0.7)
    assert np.abs(og[:, 0] - np.array(bog)).max() <= 1e-13 and abs(lg[0, 0] - blg[0]) <= 1e-13


def pin_decoder_window_independence(cache_cls, win_attn, glob_attn):
    """Changing window 1's keys and values in any chunk leaves the other windows' rows bit for bit
    unchanged; changing a cached chunk leaves the global rows unchanged."""
    window_tokens, frames, W, G, H, D = [2, 3, 2], 2, 2, 1, 2, 4
    base = _decoder_stream(cache_cls, 81, window_tokens, frames, W, G, H, D, 4)
    rows1 = np.arange(2 * 2, 2 * 2 + 2 * 3)

    def bump(c, k, v):
        k, v = k.copy(), v.copy()
        k[rows1] += 3.0
        v[rows1] -= 5.0
        return k, v
    alt = _decoder_stream(cache_cls, 81, window_tokens, frames, W, G, H, D, 4, perturb=bump)
    o0, l0 = win_attn(base[0], window_tokens, frames, base[1], 0.5, "f32")
    o1, l1 = win_attn(alt[0], window_tokens, frames, alt[1], 0.5, "f32")
    other = np.setdiff1d(np.arange(o0.shape[0]), rows1)
    assert (o0[other] == o1[other]).all() and (l0[:, other] == l1[:, other]).all()
    assert not np.allclose(o0[rows1], o1[rows1])

    def bump_cached(c, k, v):
        return (k + 1.0, v) if c == 2 else (k, v)
    alt2 = _decoder_stream(cache_cls, 81, window_tokens, frames, W, G, H, D, 4, perturb=bump_cached)
    g0, _ = glob_attn(base[0], base[2], 0.5, "f32")
    g2, _ = glob_attn(alt2[0], alt2[2], 0.5, "f32")
    assert (g0 == g2).all()


def pin_set_bank(cache_cls):
    """set_bank replaces exactly the named bank, keeps shapes, refuses a new shape."""
    r = _rng(91)
    f = lambda *s: r.standard_normal(s).astype(np.float32)
    pk, pv = f(2, 3, 2, 4), f(2, 3, 2, 4)
    c = cache_cls(pk, pv, 1)
    c.append(0, f(5, 2, 4), f(5, 2, 4))
    nk, nv = f(3, 2, 4), f(3, 2, 4)
    c.set_bank(1, nk, nv)
    k0, v0, _ = c.sequence(0)
    k1, v1, _ = c.sequence(1)
    assert (k0[:3] == pk[0]).all() and (v0[:3] == pv[0]).all()
    assert (k1[:3] == nk).all() and (v1[:3] == nv).all()
    try:
        c.set_bank(0, f(4, 2, 4), f(4, 2, 4))
    except Exception:
        pass
    else:
        raise AssertionError("a bank changed its shape")
    k0b, _, _ = c.sequence(0)
    assert (k0b[:3] == pk[0]).all()
