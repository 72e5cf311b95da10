"""The seeded input generator: determinism, its numpy specification, rounding, recipes."""
import json
import math
import os

import numpy as np
import pytest

import synth
from synth import rng, _native

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_reference_values():
    # splitmix64 with state 0: first outputs of Vigna's generator
    z = rng.splitmix64(0, 3)
    assert [int(x) for x in z] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_native_matches_numpy_spec():
    for tag in ["Q", "K", "PV"]:
        s = rng.substream_seed(123, tag, 7, 1, 0)
        a, b = rng.normal(s, 20001), _native.normal_f64(s, 20001)
        assert np.abs(a - b).max() <= 4e-16 * max(1.0, np.abs(a).max())


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.concatenate([np.random.default_rng(1).standard_normal(100000).astype(np.float32) * 100,
                        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, 1e-40, -1e-42], np.float32),
                        # exact ties: halfway between two bf16 values
                        (np.arange(1, 200, dtype=np.uint32) * 0x10000 + 0x8000).view(np.float32)])
    ours = _native.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()
    assert (rng.f32_to_bf16_bits(x) == ref).all()
    assert _native.f32_to_bf16(np.array([np.nan], np.float32))[0] == 0x7FC0


def test_normal_moments():
    x = _native.normal_f64(99, 2_000_000)
    assert abs(x.mean()) < 3e-3 and abs(x.std() - 1) < 3e-3
    assert abs((x ** 4).mean() - 3) < 0.03


def test_stream_deterministic_and_distinct():
    w = synth.get_workload("t_stream")
    a = [e["k"].copy() for e in synth.SessionStream(w)]
    b = [e["k"].copy() for e in synth.SessionStream(w)]
    assert all((x == y).all() for x, y in zip(a, b))
    assert not (a[0] == a[2]).all()


def test_ar1_chunk_process():
    w = synth.get_workload("t_stream").scaled(chunks=8)
    last = [synth.bf16_bits_to_f32(e["k"]).astype(np.float64) for e in synth.SessionStream(w) if e["step"] == 1]
    corr = [np.corrcoef(last[i].ravel(), last[i + 1].ravel())[0, 1] for i in range(len(last) - 1)]
    assert all(abs(c - 0.9) < 0.01 for c in corr), corr
    assert all(abs(x.std() - 1.0) < 0.02 for x in last)


def test_workload_shapes_golden():
    g = json.load(open(os.path.join(GOLDEN, "workload_shapes.json")))
    for res, (gw, gh, n) in g["tokens_per_frame"].items():
        W, H = map(int, res.split("x"))
        assert (W // 16, H // 16, (W // 16) * (H // 16)) == (gw, gh, n)
    for name in ["c1", "c3", "c4"]:
        w = synth.get_workload(name)
        assert (w.persistent, w.chunk, w.window, w.visible_keys) == \
            (g[name]["persistent"], g[name]["chunk"], g[name]["window"], g[name]["visible_keys"])
    assert synth.get_workload("c4").causal_block == g["c4"]["causal_block"]
    c0 = synth.get_workload("c0")
    vis = [c0.persistent + min(c, c0.window) * c0.chunk + c0.chunk for c in range(c0.chunks)]
    assert vis == g["c0"]["visible_keys_by_chunk"]


def test_boost_recipe():
    w = synth.get_workload("t_frame")
    pos = synth.workloads._boost_positions(w)
    assert len(pos) == math.floor(0.01 * w.visible_keys) and len(set(pos.tolist())) == len(pos)
    pk, pv, hist, cur = synth.single_step_inputs(w)
    K = np.concatenate([synth.bf16_bits_to_f32(pk[0])] + [synth.bf16_bits_to_f32(h[0]) for h in hist] +
                       [synth.bf16_bits_to_f32(cur[0])])
    norms = np.linalg.norm(K.reshape(K.shape[0], -1), axis=1)
    big = np.nonzero(norms > 5 * np.median(norms))[0]
    assert set(big.tolist()) == set(pos.tolist())
    g = json.load(open(os.path.join(GOLDEN, "workload_shapes.json")))
    assert math.floor(0.01 * synth.get_workload("c4").visible_keys) == g["c4"]["boosted_keys"]


def test_closed_forms_golden():
    import oracle
    g = json.load(open(os.path.join(GOLDEN, "closed_forms.json")))
    for name, case in g.items():
        if name.startswith("_"):
            continue
        n = len(case["logits"])
        # realise the logits with a 1-d query q = 1 and keys k_j = logit_j / scale
        scale = 0.25
        q = np.ones((1, 1))
        k = np.array(case["logits"])[:, None] / scale
        v = np.eye(n)
        o, lse = oracle.masked_attention(q, k, v, np.ones((1, n), bool), scale)
        # a few ulps: the logits themselves are rounded decimal expansions of ln 2, ln 3, ln 4
        assert np.abs(o[0] - np.array(case["weights"])).max() <= 4e-15
        assert abs(lse[0] - case["lse"]) <= 4e-15


def test_decoder_windows():
    """Window partition of a latent frame: every token in exactly one window, windows row-major,
    the shifted layout cut half a window earlier; the 720p decoder window's shape as the project
    page gives it (queries and keys per window, the global tokens)."""
    g = json.load(open(os.path.join(GOLDEN, "workload_shapes.json")))["decoder"]
    w = synth.get_decoder_workload("d1")
    assert [w.grid_h, w.grid_w] == g["grid_720p"] and w.window == g["window"]
    assert w.frames == g["frames_per_chunk"] and w.frames * w.window_chunks == g["cached_frames"]
    assert w.global_tokens == g["global_tokens"]
    assert w.frames * max(w.window_tokens) == g["queries_per_window"]
    assert w.global_tokens + (w.window_chunks + 1) * w.frames * max(w.window_tokens) == g["keys_per_window"]
    for name in synth.DECODER_WORKLOADS:
        d = synth.get_decoder_workload(name)
        part = d.partition()
        ix = np.concatenate(part)
        assert np.array_equal(np.sort(ix), np.arange(d.grid_h * d.grid_w)), name
        assert d.frames * sum(d.window_tokens) == d.chunk_tokens
        for p in part:   # a window is a rectangle of the grid, row-major inside
            r, c = p // d.grid_w, p % d.grid_w
            rect = ((r.min() + np.arange(r.max() - r.min() + 1))[:, None] * d.grid_w
                    + c.min() + np.arange(c.max() - c.min() + 1)[None, :]).ravel()
            assert np.array_equal(p, rect), name
            assert len(p) == (r.max() - r.min() + 1) * (c.max() - c.min() + 1)
            assert np.array_equal(p, np.sort(p))
            assert r.max() - r.min() < d.window and c.max() - c.min() < d.window
    assert synth.get_decoder_workload("d1").window_tokens == [256] * 10 + [208] * 5
    s = synth.get_decoder_workload("d1s")
    assert len(s.window_tokens) == 4 * 6 and s.window_tokens[0] == 8 * 8 and s.window_tokens[-1] == 5 * 8
    # pack_windows: window by window, frames in order inside a window
    x = np.arange(2 * 6)
    assert pack_list(synth.pack_windows(x, [np.array([0, 1, 3]), np.array([2, 4, 5])], 2, 6)) == \
        [0, 1, 3, 6, 7, 9, 2, 4, 5, 8, 10, 11]


def pack_list(a):
    return [int(v) for v in a]


def test_decoder_stream():
    """Seeded decoder chunks: packed shapes, eviction from chunk W + 1 on, fresh global tokens."""
    w = synth.get_decoder_workload("t_dec")
    evs = list(synth.DecoderStream(w))
    assert [e["evict_before"] for e in evs] == [c >= w.window_chunks + 1 for c in range(w.chunks)]
    T = w.chunk_tokens
    for e in evs:
        assert e["k"].shape == e["v"].shape == e["q"].shape == (T, w.heads, w.head_dim)
        assert e["gk"].shape == (w.global_tokens, w.heads, w.head_dim) and e["k"].dtype == np.uint16
    assert not np.array_equal(evs[0]["gk"], evs[1]["gk"])
    again = next(iter(synth.DecoderStream(w)))
    assert np.array_equal(again["k"], evs[0]["k"]) and np.array_equal(again["gq"], evs[0]["gq"])
