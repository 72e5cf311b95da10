"""GPU parity of the reduced-precision path (SR_MX: MXFP6 keys and queries, FP8 values) against
the fp64 oracle ("The road to the fastest, cheapest H3", Accelerating the denoiser, item 2).

The cache's codes must equal oracle.mx's bit for bit (through sr_kvcache_gather, which
returns the exactly representable dequantized values, and by reading the pool at the offsets
sr.h documents).  Attention results are compared element by element with the oracle's
attention over the dequantized operands, within the bound derived in gates.mx_bounds (the
kernel's one extra rounding: probabilities to FP8).
"""
import sys

import numpy as np
import pytest

import gates
import harness
import oracle
import synth
from oracle import mx as omx
from oracle.chunk_attention import current_block_mask

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sr():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return harness.lib_module()


def bf16_values(bits):
    return harness.widen_host(bits, "bf16")


def deq_k(bits):
    return omx.mxfp6_values(bf16_values(bits)).astype(np.float32)


def deq_v(bits):
    return omx.fp8_values(bf16_values(bits)).astype(np.float32)


def mx_cfg(sr, w, causal_block=None):
    return sr.config_for(w.heads, w.head_dim, w.persistent, w.chunk, w.window,
                         w.causal_block if causal_block is None else causal_block, w.banks, sr.SR_MX)


def mx_reference(model, bank, q_bits, scale, rows, causal_block=None, keys="chunk"):
    """Exact attention over the dequantized operands and its per-element bounds.
    keys: "chunk" (current rows, causal blocks), "window" (moving rows, all keys), "prefix"."""
    if keys == "prefix":                       # the bank alone; needs no current chunk
        k, v, n_fixed = model.pk[bank], model.pv[bank], model.prefix_len(bank)
    else:
        k, v, n_fixed = model.sequence(bank)
    n_cur = k.shape[0] - n_fixed
    qd = omx.mxfp6_values(bf16_values(q_bits))
    H, D = qd.shape[1], qd.shape[2]
    R = len(rows)
    o = np.zeros((R, H, D))
    lse = np.zeros((H, R))
    b_o = np.zeros((R, H, D))
    b_l = np.zeros((H, R))
    for h in range(H):
        kh, vh = k[:, h].astype(np.float64), v[:, h].astype(np.float64)
        for r0 in range(0, R, 512):
            rb = rows[r0:r0 + 512]
            if keys == "chunk":
                vis = np.concatenate([np.ones((len(rb), n_fixed), bool),
                                      current_block_mask(rb, n_cur, causal_block)], axis=1)
            else:
                vis = np.ones((len(rb), kh.shape[0]), bool)
            ob, lb, wb = oracle.masked_attention(qd[rb, h], kh, vh, vis, scale, return_probs=True)
            bo, bl = gates.mx_bounds(wb, vh, ob)
            o[r0:r0 + len(rb), h], lse[h, r0:r0 + len(rb)] = ob, lb
            b_o[r0:r0 + len(rb), h], b_l[h, r0:r0 + len(rb)] = bo, bl
    return o, lse, b_o, b_l


def run_mx_stream(sr, w, rows=None, workspace="own", check_gather=False):
    """Streams workload w into an SR_MX cache and the oracle model (which holds the dequantized
    values); every attention call is checked against mx_reference.  Returns the worst
    error / bound ratios and the plain error statistics of each checked call."""
    import torch
    scale = 1.0 / np.sqrt(w.head_dim)
    stream = synth.SessionStream(w)
    pk, pv = stream.persistent()
    cache = sr.KVCache(mx_cfg(sr, w), harness.to_dev(pk, "bf16"), harness.to_dev(pv, "bf16"), workspace=workspace)
    model = oracle.StreamingCache(deq_k(pk), deq_v(pv), w.window)
    out_stats = []
    for idx, ev in enumerate(stream):
        if ev["evict_before"]:
            assert cache.evict() == model.evict()
        cache.append(ev["chunk"], harness.to_dev(ev["k"], "bf16"), harness.to_dev(ev["v"], "bf16"))
        model.append(ev["chunk"], deq_k(ev["k"]), deq_v(ev["v"]))
        if w.single_step and ev["chunk"] != w.chunks - 1:
            continue
        n = ev["q"].shape[0]
        lse = torch.empty((w.heads, n), dtype=torch.float32, device="cuda")
        out = cache.attention(ev["bank"], harness.to_dev(ev["q"], "bf16"), lse=lse, softmax_scale=scale)
        if check_gather:
            kg, vg = cache.gather(ev["bank"])
            km, vm, _ = model.sequence(ev["bank"])
            assert (bf16_values(harness.to_host(kg, "bf16")) == km).all(), (w.name, idx, "K codes")
            assert (bf16_values(harness.to_host(vg, "bf16")) == vm).all(), (w.name, idx, "V codes")
        r = np.arange(n) if rows is None else rows[rows < n]
        o_ref, l_ref, b_o, b_l = mx_reference(model, ev["bank"], ev["q"], scale, r, w.causal_block)
        o_dev = bf16_values(harness.to_host(out, "bf16"))[r]
        ratio = gates.assert_mx(o_dev, lse.cpu().numpy()[:, r], o_ref, l_ref, b_o, b_l, (w.name, idx))
        out_stats.append((idx, ratio, gates.error_stats(o_dev, o_ref)))
    cache.close()
    return out_stats


def test_mx_codes_and_layout(sr):
    """Quantized K/V equal the oracle's codes: through gather (exact dequantized bf16) and by
    reading the pool at the offsets sr.h documents.  Inputs span subnormal to huge blocks,
    all-zero blocks, exact ties and negative zeros; two chunk lengths leave ragged pages."""
    import torch
    rng = np.random.default_rng(17)
    H, D, n = 3, 128, 300
    x = rng.standard_normal((2, n, H, D)) * np.exp2(rng.integers(-125, 120, (2, n, H, 1)).astype(np.float64))
    x = x * np.exp2(rng.uniform(-6, 0, x.shape))
    x[:, 5, 1, :32] = 0.0
    x[:, 7, 2, 40] = -0.0
    bits = synth.f32_to_bf16_bits(x.astype(np.float32))
    bits[:, 9, 0, :] = 0x8000                                     # a row of negative zeros
    bits[:, 11, 1, :] = np.array([0x0001, 0x0040, 0x807F] * 42 + [0x0001, 0x0003], np.uint16)  # bf16 subnormals
    k, v = bits[0], bits[1]
    cfg = sr.config_for(H, D, 0, n, 1, n, 1, sr.SR_MX)
    cache = sr.KVCache(cfg)
    cache.append(0, harness.to_dev(k, "bf16"), harness.to_dev(v, "bf16"))
    kg, vg = cache.gather(0)
    assert (bf16_values(harness.to_host(kg, "bf16")) == omx.mxfp6_values(bf16_values(k))).all()
    got_v = harness.to_host(vg, "bf16")
    want_v = synth.f32_to_bf16_bits(omx.fp8_values(bf16_values(v)).astype(np.float32))
    assert (got_v == want_v).all()       # bit for bit, signed zeros included
    # raw pages: codes, scale bytes and V bytes at their documented offsets (slot 0, page 0)
    pool = cache.pool.cpu().numpy()
    NB, total_pages = D // 32, (n + 127) // 128 * 2
    kpage_bytes = (NB * 3200 + 1023) // 1024 * 1024
    half = H * total_pages * kpage_bytes
    codes, X = omx.mx_quantize(bf16_values(k))
    v8 = omx.encode(bf16_values(v), omx.E4M3)
    for h in range(H):
        for t in (0, 5, 9, 11, 37, 127):
            pg = pool[h * total_pages * kpage_bytes:][:kpage_bytes]
            for b in range(NB):
                packed = np.concatenate([pg[(b * 128 + t) * 16:][:16], pg[NB * 2048 + (b * 128 + t) * 8:][:8]])
                bitsx = int.from_bytes(packed.tobytes(), "little")
                cs = [(bitsx >> (6 * e)) & 63 for e in range(32)]
                assert cs == list(codes[t, h, 32 * b:32 * b + 32]), (h, t, b)
                assert pg[NB * 3072 + t * NB + (b % 2) * (NB // 2) + b // 2] == X[t, h, b] + 127, (h, t, b)
            vp = pool[half + h * total_pages * 128 * D:][:128 * D]
            r = t % 32
            for d in (0, 31, 64, 127):
                g = 4 * (t // 64) + 2 * ((t // 32) % 2) + (r // 4) % 2
                assert vp[(g * D + d) * 16 + 4 * (r // 8) + r % 4] == v8[t, h, d], (h, t, d)
    cache.close()


SCHEDULES = {"split": "own", "whole": None}


@pytest.mark.parametrize("schedule", ["split", "whole"])
@pytest.mark.parametrize("name", ["t_stream", "t_d64", "t_frame"])
def test_mx_parity_every_element(sr, name, schedule):
    w = synth.get_workload(name)
    say(f"[mx parity] {name} ({schedule}): H={w.heads} D={w.head_dim} P={w.persistent} chunk={w.chunk} "
        f"W={w.window} cb={w.causal_block}")
    stats = run_mx_stream(sr, w, workspace=SCHEDULES[schedule], check_gather=True)
    assert stats
    worst = max(s[1][0] for s in stats)
    say(f"[mx parity] {name}: worst err/bound {worst:.3f} lse {max(s[1][1] for s in stats):.3f}; "
        f"max|err| {max(s[2]['max_abs'] for s in stats):.3g} rel_fro {max(s[2]['rel_fro'] for s in stats):.3g}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["c1", "c1s"])
def test_mx_full_size(sr, name):
    """c1 shape (24 heads x 4680 queries over 2072 + 2 x 4680 + 4680 keys) in the launch
    configuration the benchmark times (split schedule): every element of c1 (the benchmark's
    workload), sampled rows of the stress variant c1s."""
    w = synth.get_workload(name)
    rows = None if name == "c1" else harness.sample_rows(w.chunk, block=w.causal_block)
    say(f"[mx full] {name}: " + ("every row" if rows is None else f"{len(rows)} sampled rows"))
    stats = run_mx_stream(sr, w, rows=rows)
    say(f"[mx full] {name}: err/bound {stats[-1][1]}, {stats[-1][2]}")


def test_mx_window_and_prefix(sr):
    """The page-literal window calls on an SR_MX cache: moving rows over the whole window (with
    history chunks rewritten in place) and the prefix rows over their bank."""
    import torch
    w = synth.get_workload("t_win")
    scale = 1.0 / np.sqrt(w.head_dim)
    stream = synth.WindowStream(w)
    pk, pv = stream.persistent()
    cache = sr.KVCache(mx_cfg(sr, w), harness.to_dev(pk, "bf16"), harness.to_dev(pv, "bf16"))
    model = oracle.StreamingCache(deq_k(pk), deq_v(pv), w.window)
    worst = 0.0
    for b in range(w.banks):
        qp = stream.prefix_queries(b)
        lse = torch.empty((w.heads, w.persistent), dtype=torch.float32, device="cuda")
        out = cache.prefix_attention(b, harness.to_dev(qp, "bf16"), lse=lse, softmax_scale=scale)
        r = np.arange(w.persistent)
        ref = mx_reference(model, b, qp, scale, r, keys="prefix")
        worst = max(worst, gates.assert_mx(bf16_values(harness.to_host(out, "bf16")), lse.cpu().numpy(), *ref,
                                           ("prefix", b))[0])
    for idx, ev in enumerate(stream):
        if ev["evict_before"]:
            assert cache.evict() == model.evict()
        for i, k, v in ev["history"]:
            cache.update(i, harness.to_dev(k, "bf16"), harness.to_dev(v, "bf16"))
            model.update(i, deq_k(k), deq_v(v))
        cache.append(ev["chunk"], harness.to_dev(ev["k"], "bf16"), harness.to_dev(ev["v"], "bf16"))
        model.append(ev["chunk"], deq_k(ev["k"]), deq_v(ev["v"]))
        q = ev["q"]
        lse = torch.empty((w.heads, q.shape[0]), dtype=torch.float32, device="cuda")
        out = cache.window_attention(ev["bank"], harness.to_dev(q, "bf16"), lse=lse, softmax_scale=scale)
        r = np.arange(q.shape[0])
        ref = mx_reference(model, ev["bank"], q, scale, r, keys="window")
        worst = max(worst, gates.assert_mx(bf16_values(harness.to_host(out, "bf16")), lse.cpu().numpy(), *ref,
                                           ("window", idx))[0])
    say(f"[mx window] worst err/bound {worst:.3f}")
    cache.close()


def test_mx_degenerate_shapes(sr):
    """One-token chunks without persistent tokens and W = 0; a chunk of exactly one page at
    head_dim 64; ragged pages with causal blocks of half a sub-tile; a long prefix with few items
    (4 items of 69 key tiles: the fan split runs each as 8 pieces)."""
    import torch
    rng = np.random.default_rng(23)
    mk = lambda *s: synth.f32_to_bf16_bits(rng.standard_normal(s).astype(np.float32))
    for H, D, P, n, W, cb in [(2, 128, 0, 1, 0, 1), (1, 64, 5, 128, 1, 128), (3, 128, 129, 257, 2, 32),
                              (2, 128, 8000, 300, 1, 300)]:
        say(f"[mx degenerate] H={H} D={D} P={P} n={n} W={W} cb={cb}")
        pkb, pvb = mk(1, P, H, D), mk(1, P, H, D)
        cache = sr.KVCache(sr.config_for(H, D, P, n, W, cb, 1, sr.SR_MX),
                           harness.to_dev(pkb, "bf16") if P else None, harness.to_dev(pvb, "bf16") if P else None)
        model = oracle.StreamingCache(deq_k(pkb), deq_v(pvb), W)
        for c in range(4):
            if W and c > W:
                assert cache.evict() == model.evict()
            k, v, q = mk(n, H, D), mk(n, H, D), mk(n, H, D)
            cache.append(c, harness.to_dev(k, "bf16"), harness.to_dev(v, "bf16"))
            model.append(c, deq_k(k), deq_v(v))
            lse = torch.empty((H, n), dtype=torch.float32, device="cuda")
            out = cache.attention(0, harness.to_dev(q, "bf16"), lse=lse, softmax_scale=0.125)
            ref = mx_reference(model, 0, q, 0.125, np.arange(n), causal_block=cb)
            gates.assert_mx(bf16_values(harness.to_host(out, "bf16")), lse.cpu().numpy(), *ref, (H, D, P, n, c))
        cache.close()


def test_mx_queue_split_uneven_xcds(sr):
    """The queue split on an SR_MX cache with 260 items (20 heads x 13 query tiles at head_dim
    64): XCDs own 32 or 33 items, so half of them have one split item and half none."""
    import torch
    rng = np.random.default_rng(29)
    mk = lambda *s: synth.f32_to_bf16_bits(rng.standard_normal(s).astype(np.float32))
    H, D, n, W = 20, 64, 3300, 2
    say(f"[mx queue edge] H={H} D={D} n={n} W={W}")
    cache = sr.KVCache(sr.config_for(H, D, 0, n, W, n, 1, sr.SR_MX), None, None)
    none = mk(1, 0, H, D)
    model = oracle.StreamingCache(deq_k(none), deq_v(none), W)
    for c in range(W + 1):
        k, v = mk(n, H, D), mk(n, H, D)
        cache.append(c, harness.to_dev(k, "bf16"), harness.to_dev(v, "bf16"))
        model.append(c, deq_k(k), deq_v(v))
    q = mk(n, H, D)
    lse = torch.empty((H, n), dtype=torch.float32, device="cuda")
    out = cache.attention(0, harness.to_dev(q, "bf16"), lse=lse, softmax_scale=0.125)
    ref = mx_reference(model, 0, q, 0.125, np.arange(n), causal_block=n)
    ratio = gates.assert_mx(bf16_values(harness.to_host(out, "bf16")), lse.cpu().numpy(), *ref, ("queue", H, n))
    say(f"[mx queue edge] err/bound {ratio}")
    cache.close()


def test_mx_call_errors(sr):
    """The fused qkv append is not offered on SR_MX caches; the ring stays as it was."""
    import torch
    H, D, n = 2, 128, 64
    cache = sr.KVCache(sr.config_for(H, D, 0, n, 1, n, 1, sr.SR_MX))
    qkv = torch.zeros((n, 3, H, D), dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros((n, 3), dtype=torch.int32, device="cuda")
    g = torch.ones(D, dtype=torch.float32, device="cuda")
    with pytest.raises(sr.SrError) as e:
        cache.append_qkv(0, qkv, pos, g, g, sr.qk_prep((16, 24, 24)))
    assert e.value.status == 5
    with pytest.raises(sr.SrError) as e:
        cache.segments()                  # still no current chunk
    assert e.value.status == 2
    cache.close()
