"""GPU parity of the streaming decoder's window attention against the fp64 oracle.

A windowed cache (sr_kvcache_set_window_layout) streams chunks of latent frames packed window by
window (sr_kvcache_append_windows), rewrites the global tokens every chunk (sr_kvcache_set_bank),
and runs every window's attention in one launch (sr_windows_attention) and the global tokens'
attention to the whole chunk (sr_global_attention, split-K with a workspace), all through the C
ABI.  Every element at the 720p decoder shape and on reduced streams, both window layouts
(plain and shifted), with the gathered cache bit-exact against the oracle's cache model.
Gates: tests/gates.py.
"""
import sys

import numpy as np
import pytest

import gates
import harness
import oracle
import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sr():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return harness.lib_module()


def decoder_cache(sr, w, workspace="own"):
    dt = sr.SR_BF16 if w.dtype == "bf16" else sr.SR_F32
    cfg = sr.config_for(w.heads, w.head_dim, w.global_tokens, w.capacity, w.window_chunks, w.capacity, 1, dt)
    z = np.zeros((1, w.global_tokens, w.heads, w.head_dim), dtype=np.uint16 if w.dtype == "bf16" else np.float32)
    cache = sr.KVCache(cfg, harness.to_dev(z, w.dtype), harness.to_dev(z, w.dtype), workspace=workspace)
    cache.set_window_layout(w.window_tokens, w.frames, w.window_pages)
    return cache, oracle.StreamingCache(z, z, w.window_chunks)


def run_decoder_stream(sr, w, workspace="own", check_gather=True):
    """Streams decoder workload `w` through the library and the oracle model; returns the error
    statistics of every chunk's window and global attention."""
    import torch
    scale = 1.0 / np.sqrt(w.head_dim)
    cache, model = decoder_cache(sr, w, workspace)
    T, G = w.chunk_tokens, w.global_tokens
    stats = []
    for ev in synth.DecoderStream(w):
        c = ev["chunk"]
        if ev["evict_before"]:
            assert cache.evict() == model.evict()
        cache.set_bank(0, harness.to_dev(ev["gk"], w.dtype), harness.to_dev(ev["gv"], w.dtype))
        model.set_bank(0, ev["gk"], ev["gv"])
        cache.append_windows(c, harness.to_dev(ev["k"], w.dtype), harness.to_dev(ev["v"], w.dtype))
        model.append(c, ev["k"], ev["v"])
        lse = torch.full((w.heads, T), float("nan"), dtype=torch.float32, device="cuda")
        out = cache.windows_attention(0, harness.to_dev(ev["q"], w.dtype), lse=lse, softmax_scale=scale)
        glse = torch.full((w.heads, G), float("nan"), dtype=torch.float32, device="cuda")
        gout = cache.global_attention(0, harness.to_dev(ev["gq"], w.dtype), lse=glse, softmax_scale=scale)
        if check_gather:
            kg, vg = cache.gather(0)
            km, vm, _ = model.sequence(0)
            assert (harness.to_host(kg, w.dtype) == km).all() and (harness.to_host(vg, w.dtype) == vm).all(), \
                (w.name, c)
        o_ref, l_ref = oracle.decoder_window_attention(model, w.window_tokens, w.frames, ev["q"], scale, w.dtype)
        g_ref, gl_ref = oracle.decoder_global_attention(model, ev["gq"], scale, w.dtype)
        out_h = harness.widen_host(harness.to_host(out, w.dtype), w.dtype)
        gout_h = harness.widen_host(harness.to_host(gout, w.dtype), w.dtype)
        lse_h, glse_h = lse.cpu().numpy(), glse.cpu().numpy()
        assert np.isfinite(out_h).all() and np.isfinite(lse_h).all(), (w.name, c)
        assert np.isfinite(gout_h).all() and np.isfinite(glse_h).all(), (w.name, c)
        stats.append((("windows", c), gates.error_stats(out_h, o_ref), gates.error_stats(lse_h, l_ref)))
        stats.append((("global", c), gates.error_stats(gout_h, g_ref), gates.error_stats(glse_h, gl_ref)))
    cache.close()
    return stats


def check_stats(w, stats):
    g = gates.gates_for(w.dtype)
    lse_tol = 2e-2 if w.dtype == "bf16" else 1e-4
    for what, st, st_l in stats:
        assert gates.passes(st, g), (w.name, what, st)
        assert st_l["max_abs"] <= lse_tol, (w.name, what, st_l)


@pytest.mark.parametrize("schedule", ["split", "whole"])
@pytest.mark.parametrize("name", ["t_dec", "t_dec_s", "t_dec64", "t_decf32", "t_decmax"])
def test_decoder_parity_every_element(sr, name, schedule):
    w = synth.get_decoder_workload(name)
    say(f"[decoder] {name} ({schedule}): H={w.heads} D={w.head_dim} windows={len(w.window_tokens)} "
        f"tokens={sorted(set(w.window_tokens))} frames={w.frames} W={w.window_chunks} G={w.global_tokens}")
    stats = run_decoder_stream(sr, w, workspace="own" if schedule == "split" else None)
    assert len(stats) == 2 * w.chunks
    check_stats(w, stats)
    say(f"[decoder] {name}: worst", max(s[1]["max_abs"] for s in stats), max(s[1]["rel_fro"] for s in stats))


@pytest.mark.parametrize("name", ["d1", "d1s"])
def test_decoder_full_size_every_element(sr, name):
    """720p decoder layer: 15 windows (or 24 shifted) of up to 512 queries over 5 + 3 x 512 keys,
    16 heads, four chunks (the last after an eviction); every output element."""
    w = synth.get_decoder_workload(name)
    say(f"[decoder full] {name}: {len(w.window_tokens)} windows, T={w.chunk_tokens}")
    stats = run_decoder_stream(sr, w, check_gather=(name == "d1"))
    check_stats(w, stats)
    say(f"[decoder full] {name}:", stats[-2][1], "global", stats[-1][1])


def test_decoder_windows_are_independent(sr):
    """Changing one window's keys of a history chunk moves that window's rows only, bit for bit;
    the global rows see the current chunk only, so they do not move either."""
    import torch
    w = synth.get_decoder_workload("t_dec")
    scale = 1.0 / np.sqrt(w.head_dim)
    evs = list(synth.DecoderStream(w))[:2]
    outs = []
    for poke in (False, True):
        cache, _ = decoder_cache(sr, w, None)
        for ev in evs:
            k = ev["k"].copy()
            if poke and ev["chunk"] == 0:
                rows = oracle.decoder.window_rows(w.window_tokens, w.frames, 3)
                k[rows] = ev["k"][rows[::-1]]
            cache.set_bank(0, harness.to_dev(ev["gk"], w.dtype), harness.to_dev(ev["gv"], w.dtype))
            cache.append_windows(ev["chunk"], harness.to_dev(k, w.dtype), harness.to_dev(ev["v"], w.dtype))
        q = harness.to_dev(evs[-1]["q"], w.dtype)
        o = cache.windows_attention(0, q, softmax_scale=scale)
        go = cache.global_attention(0, harness.to_dev(evs[-1]["gq"], w.dtype), softmax_scale=scale)
        torch.cuda.synchronize()
        outs.append((harness.to_host(o, w.dtype), harness.to_host(go, w.dtype)))
        cache.close()
    rows = oracle.decoder.window_rows(w.window_tokens, w.frames, 3)
    other = np.setdiff1d(np.arange(w.chunk_tokens), rows)
    assert np.array_equal(outs[0][0][other], outs[1][0][other])
    assert not np.array_equal(outs[0][0][rows], outs[1][0][rows])
    assert np.array_equal(outs[0][1], outs[1][1])


def test_decoder_call_errors(sr):
    """Window calls need a layout; contiguous calls are refused on a windowed cache; layouts that
    do not fit a slot, or come after the first append, are refused and change nothing."""
    import torch
    rng = np.random.default_rng(11)
    H, D, G, cap = 2, 128, 5, 4 * 128
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s).astype(np.float32)).to(torch.bfloat16).cuda()
    gk, gv = mk(1, G, H, D), mk(1, G, H, D)
    cache = sr.KVCache(sr.config_for(H, D, G, cap, 1, cap, 1, sr.SR_BF16), gk, gv)
    T = 2 * (64 + 100)
    k, v, q = mk(T, H, D), mk(T, H, D), mk(T, H, D)
    out = torch.empty_like(q)
    for call in (lambda: sr.sr_windows_attention(cache.h, 0, q, out),
                 lambda: sr.sr_global_attention(cache.h, 0, q[:G], out[:G]),
                 lambda: sr.sr_kvcache_append_windows(cache.h, 0, k, v)):
        with pytest.raises(sr.SrError) as e:
            call()
        assert e.value.status == 2                          # no layout
    for tok, frames, pages in (([], 2, 1), ([64, 100, 1], 2, 1), ([64, 100], 2, 3), ([65, 100], 2, 1),
                               ([0, 100], 2, 1), ([64, 100], 0, 1), ([64, 100], 2, 0)):
        with pytest.raises(sr.SrError) as e:
            sr.sr_kvcache_set_window_layout(cache.h, sr.window_layout(tok, frames, pages))
        assert e.value.status == 1, (tok, frames, pages)
    cache.set_window_layout([64, 100], 2, 2)
    with pytest.raises(sr.SrError) as e:
        cache.set_window_layout([64, 100], 2, 2)
    assert e.value.status == 2                              # once only
    with pytest.raises(sr.SrError) as e:
        cache.windows_attention(0, q)
    assert e.value.status == 2                              # no current chunk
    with pytest.raises(ValueError):
        cache.append_windows(0, k[:-1], v[:-1])             # packed rows must be T
    cache.append_windows(0, k, v)
    with pytest.raises(ValueError):
        cache.windows_attention(0, q[:-1])
    for call, args in ((cache.append, (1, k, v)), (cache.update, (0, k, v)), (cache.attention, (0, q)),
                       (cache.window_attention, (0, q)), (cache.prefix_attention, (0, q[:G]))):
        with pytest.raises(sr.SrError) as e:
            call(*args)
        assert e.value.status == 2, call
    with pytest.raises(sr.SrError) as e:
        sr.sr_kvcache_set_bank(cache.h, 1, gk[0], gv[0])
    assert e.value.status == 1                              # bank out of range
    with pytest.raises(sr.SrError) as e:
        sr.sr_global_attention(cache.h, 0, q[:G], out[:G], softmax_scale=0.0)
    assert e.value.status == 1
    o = cache.windows_attention(0, q)
    go = cache.global_attention(0, q[:G])
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(go.float()).all()
    cache.close()
    mx = sr.KVCache(sr.config_for(H, D, G, cap, 1, cap, 1, sr.SR_MX), gk, gv)
    with pytest.raises(sr.SrError) as e:
        mx.set_window_layout([64, 100], 2, 2)
    assert e.value.status == 5                              # SR_MX: not with a window layout
    mx.close()
    nog = sr.KVCache(sr.config_for(H, D, 0, cap, 1, cap, 1, sr.SR_BF16))
    with pytest.raises(sr.SrError) as e:
        sr.sr_kvcache_set_bank(nog.h, 0, gk[0], gv[0])
    assert e.value.status == 1                              # no persistent tokens
    nog.close()


@pytest.mark.parametrize("workspace", ["own", None])
def test_decoder_without_global_tokens(sr, workspace):
    """A windowed cache with no persistent tokens: each window over its own keys only, the
    global call over the current chunk only (the few-row kernel with a workspace, the chunk
    kernel without); every element against the oracle."""
    import torch
    rng = np.random.default_rng(12)
    H, D, cap, tok, frames = 2, 128, 6 * 128, [64, 100, 7], 2
    T = frames * sum(tok)
    bf = lambda *s: synth.f32_to_bf16_bits(rng.standard_normal(s).astype(np.float32))
    cache = sr.KVCache(sr.config_for(H, D, 0, cap, 2, cap, 1, sr.SR_BF16), workspace=workspace)
    cache.set_window_layout(tok, frames, 2)
    z = np.zeros((1, 0, H, D), dtype=np.uint16)
    model = oracle.StreamingCache(z, z, 2)
    scale = 1.0 / np.sqrt(D)
    for c in range(3):
        k, v, q, gq = bf(T, H, D), bf(T, H, D), bf(T, H, D), bf(3, H, D)
        cache.append_windows(c, harness.to_dev(k, "bf16"), harness.to_dev(v, "bf16"))
        model.append(c, k, v)
        lse = torch.full((H, T), float("nan"), dtype=torch.float32, device="cuda")
        o = cache.windows_attention(0, harness.to_dev(q, "bf16"), lse=lse, softmax_scale=scale)
        go = cache.global_attention(0, harness.to_dev(gq, "bf16"), softmax_scale=scale)
        o_ref, l_ref = oracle.decoder_window_attention(model, tok, frames, q, scale, "bf16")
        g_ref, _ = oracle.decoder_global_attention(model, gq, scale, "bf16")
        gates.assert_gates(harness.widen_host(harness.to_host(o, "bf16"), "bf16"), o_ref, "bf16", f"windows {c}")
        gates.assert_gates(harness.widen_host(harness.to_host(go, "bf16"), "bf16"), g_ref, "bf16", f"global {c}")
        assert np.abs(lse.cpu().numpy() - l_ref).max() <= 2e-2
    cache.close()


@pytest.mark.parametrize("head_dim", [128, 64])
def test_global_attention_row_counts(sr, head_dim):
    """Global-token attention for 1 to 33 query rows (32 is the most the few-row split-K kernel
    takes; 33 runs the chunk-attention kernel), with and without a workspace, against the oracle;
    a second call gives the same bits (the arrival counters are left at zero)."""
    import torch
    rng = np.random.default_rng(13 + head_dim)
    H, G, tok, frames = 3, 5, [64, 100, 7, 64], 2
    cap = len(tok) * 2 * 128
    T = frames * sum(tok)
    bf = lambda *s: synth.f32_to_bf16_bits(rng.standard_normal(s).astype(np.float32))
    gk, gv = bf(1, G, H, head_dim), bf(1, G, H, head_dim)
    model = oracle.StreamingCache(gk, gv, 1)
    k, v = bf(T, H, head_dim), bf(T, H, head_dim)
    model.append(0, k, v)
    scale = 1.0 / np.sqrt(head_dim)
    for ws in ("own", None):
        cache = sr.KVCache(sr.config_for(H, head_dim, G, cap, 1, cap, 1, sr.SR_BF16),
                           harness.to_dev(gk, "bf16"), harness.to_dev(gv, "bf16"), workspace=ws)
        cache.set_window_layout(tok, frames, 2)
        cache.append_windows(0, harness.to_dev(k, "bf16"), harness.to_dev(v, "bf16"))
        for n in (1, 5, 31, 32, 33):
            gq = bf(n, H, head_dim)
            lse = torch.full((H, n), float("nan"), dtype=torch.float32, device="cuda")
            o = cache.global_attention(0, harness.to_dev(gq, "bf16"), lse=lse, softmax_scale=scale)
            o2 = cache.global_attention(0, harness.to_dev(gq, "bf16"), softmax_scale=scale)
            torch.cuda.synchronize()
            assert torch.equal(o, o2), (ws, n)
            g_ref, l_ref = oracle.decoder_global_attention(model, gq, scale, "bf16")
            gates.assert_gates(harness.widen_host(harness.to_host(o, "bf16"), "bf16"), g_ref, "bf16", f"{ws} {n}")
            assert np.abs(lse.cpu().numpy() - l_ref).max() <= 2e-2, (ws, n)
        cache.close()
