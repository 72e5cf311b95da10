"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

The reference is the plain C++ fp64 oracle (oracle/native.py; cross-checked against the numpy
oracle on the CPU).  Every element on reduced workloads that span several query and key tiles
with ragged tails, and every element at the full workload sizes in the launch configuration
the benchmark times (the split schedule; c1 and c4 also with whole items).  The 64-step c2
session is checked whole on its first six and last two chunk-steps, on sampled rows in
between, with a bit-exact gather of both banks after every step.  Gates: tests/gates.py.
"""
import sys

import numpy as np
import pytest

import gates
import harness
import synth
from oracle import native

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sr():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return harness.lib_module()


def run_stream(sr, w, phase=0, rows=None, check_gather=False, oracle_every=1, on_step=None, workspace="own",
               whole_steps=None):
    """Streams workload `w` through the library and the oracle's cache model; returns per-step
    stats (step index, output stats, lse stats).  workspace "own": the split schedule (the
    default a KVCache runs); None: one workgroup per item.  rows: rows checked (None: all);
    whole_steps: step indices checked on every row whatever `rows` says."""
    import torch
    scale = 1.0 / np.sqrt(w.head_dim)
    stream = synth.SessionStream(w)
    pk, pv = stream.persistent()
    cache = sr.KVCache(harness.cfg_of(sr, w), harness.to_dev(pk, w.dtype), harness.to_dev(pv, w.dtype),
                       workspace=workspace)
    model = native.StreamingCache(pk, pv, w.window)
    stats = []
    for idx, ev in enumerate(stream):
        cid = ev["chunk"] + phase
        if ev["evict_before"]:
            assert cache.evict() == model.evict()
        cache.append(cid, harness.to_dev(ev["k"], w.dtype), harness.to_dev(ev["v"], w.dtype))
        model.append(cid, ev["k"], ev["v"])
        if w.single_step and ev["chunk"] != w.chunks - 1:
            continue
        q = harness.to_dev(ev["q"], w.dtype)
        lse = torch.empty((w.heads, w.chunk), dtype=torch.float32, device="cuda")
        out = cache.attention(ev["bank"], q, lse=lse, softmax_scale=scale)
        if check_gather:
            for b in range(w.banks):
                kg, vg = cache.gather(b)
                km, vm, _ = model.sequence(b)
                assert (harness.to_host(kg, w.dtype) == km).all() and (harness.to_host(vg, w.dtype) == vm).all(), \
                    (w.name, phase, idx, b)
        out_h = harness.to_host(out, w.dtype)
        lse_h = lse.cpu().numpy()
        if on_step:
            on_step(idx, ev, out_h, lse_h)
        if idx % oracle_every and not (w.single_step):
            continue
        r = np.arange(w.chunk) if rows is None or (whole_steps and idx in whole_steps) else rows
        o_ref, l_ref = native.chunk_attention(model, ev["bank"], ev["q"], scale, w.causal_block, w.dtype, rows=r)
        o_dev = harness.widen_host(out_h[r], w.dtype)
        st = gates.error_stats(o_dev, o_ref)
        st_l = gates.error_stats(lse_h[:, r], l_ref)
        assert np.isfinite(harness.widen_host(out_h, w.dtype)).all()
        stats.append((idx, st, st_l))
    cache.close()
    return stats


def check_stats(w, stats):
    g = gates.gates_for(w.dtype)
    lse_tol = 2e-2 if w.dtype == "bf16" else 1e-4
    for idx, st, st_l in stats:
        assert gates.passes(st, g), (w.name, idx, st)
        assert st_l["max_abs"] <= lse_tol, (w.name, idx, st_l)


SCHEDULES = {"split": "own", "whole": None}


@pytest.mark.parametrize("schedule", ["split", "whole"])
@pytest.mark.parametrize("name", ["c0", "t_f32", "t_stream", "t_d64", "t_frame"])
def test_parity_every_element(sr, name, schedule):
    w = synth.get_workload(name)
    say(f"[parity] {name} ({schedule}): H={w.heads} D={w.head_dim} P={w.persistent} chunk={w.chunk} W={w.window}")
    stats = run_stream(sr, w, check_gather=True, workspace=SCHEDULES[schedule])
    assert stats
    check_stats(w, stats)
    say(f"[parity] {name}: worst", max(s[1]["max_abs"] for s in stats), max(s[1]["rel_fro"] for s in stats))


@pytest.mark.parametrize("name", ["c0", "t_stream"])
def test_ring_phase_bit_identical(sr, name):
    """Same stream started at chunk id 0, 100 and 1000: same bits (slots differ)."""
    w = synth.get_workload(name)
    outs = {}
    for phase in (0, 100, 1000):
        say(f"[phase] {name} phase {phase}")
        got = []
        run_stream(sr, w, phase=phase, rows=np.arange(2), check_gather=(phase != 0),
                   on_step=lambda i, ev, o, l: got.append((o.copy(), l.copy())))
        outs[phase] = got
    for phase in (100, 1000):
        for (a, la), (b, lb) in zip(outs[0], outs[phase]):
            assert (a == b).all() and (la == lb).all()


FULL = ["c1", "c3", "c4", "c1s", "c4s"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_parity_full_size_every_element(sr, name):
    """One chunk-step at the workload's full size, every row of every head (O and LSE), in the
    benchmark's launch configuration (split schedule) and, for c1 and c4, with whole items too.
    The oracle's result is computed once and serves both schedules."""
    import time
    import torch
    w = synth.get_workload(name)
    scale = 1.0 / np.sqrt(w.head_dim)
    pk, pv, hist, cur = synth.single_step_inputs(w)
    schedules = ["split", "whole"] if name in ("c1", "c4") else ["split"]
    say(f"[full] {name}: {w.chunk} rows x {w.heads} heads over {w.visible_keys} keys, schedules {schedules}")
    outs = {}
    for sch in schedules:
        cache = sr.KVCache(harness.cfg_of(sr, w), harness.to_dev(pk, w.dtype), harness.to_dev(pv, w.dtype),
                           workspace=SCHEDULES[sch])
        for i, (k, v) in enumerate(hist):
            cache.append(i, harness.to_dev(k, w.dtype), harness.to_dev(v, w.dtype))
        cache.append(len(hist), harness.to_dev(cur[0], w.dtype), harness.to_dev(cur[1], w.dtype))
        lse = torch.empty((w.heads, w.chunk), dtype=torch.float32, device="cuda")
        out = cache.attention(0, harness.to_dev(cur[2], w.dtype), lse=lse, softmax_scale=scale)
        outs[sch] = (harness.widen_host(harness.to_host(out, w.dtype), w.dtype), lse.cpu().numpy())
        cache.close()
    model = native.StreamingCache(pk, pv, w.window)
    for i, (k, v) in enumerate(hist):
        model.append(i, k, v)
    model.append(len(hist), cur[0], cur[1])
    t0 = time.perf_counter()
    o_ref, l_ref = native.chunk_attention(model, 0, cur[2], scale, w.causal_block, w.dtype)
    say(f"[full] {name}: oracle {time.perf_counter() - t0:.1f} s")
    g = gates.gates_for(w.dtype)
    for sch, (o, l) in outs.items():
        assert np.isfinite(o).all() and np.isfinite(l).all()
        st, st_l = gates.error_stats(o, o_ref), gates.error_stats(l, l_ref)
        say(f"[full] {name} ({sch}): max {st['max_abs']:.3g} mean {st['mean_abs']:.3g} rel {st['rel_fro']:.3g} "
            f"lse max {st_l['max_abs']:.3g}")
        assert gates.passes(st, g), (name, sch, st)
        assert st_l["max_abs"] <= 2e-2, (name, sch, st_l)


def test_one_gpu_share_of_sharded_run(sr):
    """c1 shapes with 3 heads (one GPU's share when 24 heads are sharded over 8): 57 items,
    fewer than the compute units, so the workspace runs each as 4 equal pieces (fan split)."""
    w = synth.get_workload("c1").scaled(heads=3)
    rows = harness.sample_rows(w.chunk)
    say(f"[share] c1 x 3 heads: {len(rows)} sampled rows")
    stats = run_stream(sr, w, rows=rows)
    check_stats(w, stats)


def test_split_schedule_is_deterministic_and_leaves_counters_zero(sr):
    """Repeated calls give the same bits whichever piece merges; a workspace shared by two
    caches works; the arrival and queue counters are zero after every call; split and whole schedules
    agree within rounding."""
    import torch
    w = synth.get_workload("t_stream")
    cfg = harness.cfg_of(sr, w)
    ws = sr.workspace_for(cfg)
    pk, pv, hist, cur = synth.single_step_inputs(w)
    caches = []
    for workspace in (ws, ws, None):
        c = sr.KVCache(cfg, harness.to_dev(pk, w.dtype), harness.to_dev(pv, w.dtype), workspace=workspace)
        for i, (k, v) in enumerate(hist):
            c.append(i, harness.to_dev(k, w.dtype), harness.to_dev(v, w.dtype))
        c.append(len(hist), harness.to_dev(cur[0], w.dtype), harness.to_dev(cur[1], w.dtype))
        caches.append(c)
    q = harness.to_dev(cur[2], w.dtype)
    outs = [caches[i % 2].attention(0, q) for i in range(6)]
    whole = caches[2].attention(0, q)
    torch.cuda.synchronize()
    first = harness.to_host(outs[0], w.dtype)
    for o in outs[1:]:
        assert (harness.to_host(o, w.dtype) == first).all()
    # the arrival and queue counters (8 C + 16 int32 with C = CUs / 8, padded to 256 bytes)
    # end the workspace
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    counters = ws[ws.numel() - ((8 * max(cus // 8, 1) + 16) * 4 + 255) // 256 * 256:].view(torch.int32)
    assert int(counters.abs().sum()) == 0
    st = gates.error_stats(harness.widen_host(first, w.dtype),
                           harness.widen_host(harness.to_host(whole, w.dtype), w.dtype))
    assert st["max_abs"] <= 2e-2 and st["rel_fro"] <= 1e-2, st
    for c in caches:
        c.close()


@pytest.mark.timeout(900)
def test_session_c2(sr):
    """32 chunks x 2 steps with per-step banks and evictions: every element of the first six
    chunk-steps (the window filling, the first eviction) and of the last two, sampled rows of
    the others, and after every step a bit-exact gather of both banks' logical sequences."""
    w = synth.get_workload("c2")
    rows = harness.sample_rows(w.chunk, stride=211)
    whole = {0, 1, 2, 3, 4, 5, 62, 63}
    say(f"[c2] 64 chunk-steps: whole outputs at {sorted(whole)}, {len(rows)} rows at the others, gather every step")
    stats = run_stream(sr, w, rows=rows, check_gather=True, whole_steps=whole)
    assert len(stats) == 64
    check_stats(w, stats)
    errs = [s[1]["rel_fro"] for s in stats]
    say("[c2] rel_fro first/last/max", errs[0], errs[-1], max(errs))
    # no drift with the chunk index: the last steps are no worse than twice the first steps
    assert np.mean(errs[-8:]) <= 2 * np.mean(errs[:8]) + 1e-4


def _one_chunk_cache(sr, H, D, P, n, W, cb, dtype, seed, cap=None):
    import torch
    rng = np.random.default_rng(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cfg = sr.config_for(H, D, P, cap or n, W, cb, 1, sr.SR_BF16 if dtype == "bf16" else sr.SR_F32)
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s).astype(np.float32)).to(tdt).cuda()
    pk, pv = (mk(1, P, H, D), mk(1, P, H, D)) if P else (None, None)
    cache = sr.KVCache(cfg, pk, pv)
    return cache, mk, pk, pv


def test_single_visible_key_is_exact(sr):
    """With causal blocks of one token, no prefix and no history, query 0 sees only key 0:
    its output is V[0] bit for bit, and its lse is its own scaled logit."""
    import torch
    for dtype, D in (("bf16", 128), ("bf16", 64), ("f32", 64)):
        cache, mk, _, _ = _one_chunk_cache(sr, 3, D, 0, 70, 0, 1, dtype, 1)
        k, v, q = mk(70, 3, D), mk(70, 3, D), mk(70, 3, D)
        cache.append(5, k, v)
        lse = torch.empty((3, 70), dtype=torch.float32, device="cuda")
        out = cache.attention(0, q, lse=lse, softmax_scale=0.1)
        assert torch.equal(out[0], v[0]), dtype
        s0 = (q[0].float() * k[0].float()).sum(-1) * 0.1
        assert torch.allclose(lse[:, 0], s0, atol=1e-5, rtol=1e-5)
        cache.close()


def test_equal_scores_give_mean(sr):
    import torch
    cache, mk, pk, pv = _one_chunk_cache(sr, 2, 128, 100, 300, 1, 300, "bf16", 2)
    k, v = mk(300, 2, 128), mk(300, 2, 128)
    cache.append(0, k, v)
    q = torch.zeros((300, 2, 128), dtype=torch.bfloat16, device="cuda")
    out = cache.attention(0, q).float()
    mean = torch.cat([pv[0], v]).float().mean(0)
    assert (out - mean[None]).abs().max().item() <= 4e-3  # one bf16 rounding of a value < 0.3
    cache.close()


def test_hidden_data_does_not_matter(sr):
    """Bits of the output do not change when data the kernel must not read changes:
    an evicted chunk's slot, the zero tail of a short chunk, later causal blocks."""
    import torch
    H, D, P, cap, W = 2, 128, 150, 400, 2
    cache, mk, _, _ = _one_chunk_cache(sr, H, D, P, 0, W, 130, "bf16", 3, cap=cap)
    n = 333                                    # short current chunk: the tail of its slot is padding
    cache.append(0, mk(cap, H, D), mk(cap, H, D))
    cache.append(1, mk(cap, H, D), mk(cap, H, D))
    k2, v2 = mk(n, H, D), mk(n, H, D)
    cache.append(2, k2, v2)
    assert cache.evict() == 0                  # chunk 0's slot (slot 0) is now free
    q = mk(n, H, D)
    ref = cache.attention(0, q).clone()
    pool = cache.pool.view(torch.bfloat16)
    half = pool.numel() // 2
    total_pages = cache.bytes // (2 * H * 128 * D * 2)
    ppb, pps = -(-P // 128), -(-cap // 128)
    slot_page = lambda s: ppb + s * pps
    segs = cache.segments(0)
    assert [sg[0] for sg in segs] == [-1, 1, 2] and segs[-1][3] == slot_page(2)
    # 1) garbage in the evicted chunk's slot (K rows and V^T pages of every head)
    for h in range(H):
        for part in (0, half):
            p0 = part + (h * total_pages + slot_page(0)) * 128 * D
            pool[p0:p0 + pps * 128 * D] = 3.0
    torch.cuda.synchronize()
    assert torch.equal(cache.attention(0, q), ref)
    # 2) finite garbage in the padding past the current chunk's 333 tokens.  Page layout:
    #    K [D/8][128 rows, permuted in blocks of 32][8], V [128/8][D][8 tokens].
    def row(t):
        r = t & 31
        return (t & ~31) | (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1)
    pad = list(range(n % 128, 128))
    for h in range(H):
        kp = (h * total_pages + slot_page(2) + n // 128) * 128 * D
        kpage = pool[kp:kp + 128 * D].view(D // 8, 128, 8)
        kpage[:, [row(t) for t in pad], :] = -5.0
        vpage = pool[half + kp:half + kp + 128 * D].view(128 // 8, D, 8)
        for t in pad:
            vpage[t // 8, :, t % 8] = 7.0
    torch.cuda.synchronize()
    assert torch.equal(cache.attention(0, q), ref)
    # 3) later causal blocks: change keys/values of blocks >= 2 (tokens 260..332)
    k3, v3 = k2.clone(), v2.clone()
    k3[260:] = 2.0
    v3[260:] = -1.0
    cache.append(2, k3, v3)
    out3 = cache.attention(0, q)
    assert torch.equal(out3[:260], ref[:260]) and not torch.equal(out3[260:], ref[260:])
    cache.close()


def _stream_vs_oracle(sr, H, D, P, cap, W, cb, dtype, seed, chunks, workspace, rows=None):
    """Streams chunks of the given lengths (evicting when the window is full) through a device
    cache and the oracle's cache model, then checks the last chunk's attention element by
    element (or on `rows`) against the oracle."""
    import torch
    rng = np.random.default_rng(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def draw(*shape):
        t = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(tdt)
        return t, harness.to_host(t.cuda(), dtype)

    cfg = sr.config_for(H, D, P, cap, W, cb, 1, sr.SR_BF16 if dtype == "bf16" else sr.SR_F32)
    pk_t, pk = draw(1, P, H, D)
    pv_t, pv = draw(1, P, H, D)
    cache = sr.KVCache(cfg, pk_t.cuda() if P else None, pv_t.cuda() if P else None, workspace=workspace)
    model = native.StreamingCache(pk, pv, W)
    for cid, n in enumerate(chunks):
        if W > 0 and cid >= W + 1:
            assert cache.evict() == model.evict()
        (k_t, k), (v_t, v) = draw(n, H, D), draw(n, H, D)
        cache.append(cid, k_t.cuda(), v_t.cuda())
        model.append(cid, k, v)
    q_t, q = draw(chunks[-1], H, D)
    scale = 1.0 / np.sqrt(D)
    lse = torch.empty((H, chunks[-1]), dtype=torch.float32, device="cuda")
    out = cache.attention(0, q_t.cuda(), lse=lse, softmax_scale=scale)
    r = np.arange(chunks[-1]) if rows is None else rows
    o_ref, l_ref = native.chunk_attention(model, 0, q, scale, cb, dtype, rows=r)
    st = gates.error_stats(harness.widen_host(harness.to_host(out, dtype)[r], dtype), o_ref)
    assert gates.passes(st, gates.gates_for(dtype)), st
    assert np.abs(lse.cpu().numpy()[:, r] - l_ref).max() <= (2e-2 if dtype == "bf16" else 1e-4)
    cache.close()
    return st


EDGE = [  # H, D, P, cap, W, cb, dtype, chunks
    ("one key, no prefix or history", 2, 128, 0, 1, 0, 1, "bf16", [1]),
    ("fully causal blocks", 2, 128, 0, 300, 0, 1, "bf16", [300]),
    ("fully causal, fp32", 2, 64, 0, 200, 0, 1, "f32", [200]),
    ("one head, ragged pages", 1, 64, 5, 129, 1, 129, "bf16", [129, 129, 129]),
    ("short chunk in a large slot", 2, 128, 300, 1000, 2, 1000, "bf16", [1000, 1000, 3]),
    ("one-token history chunks", 3, 128, 7, 40, 3, 17, "bf16", [1, 1, 1, 40]),
    ("no prefix, full window", 2, 64, 0, 256, 3, 64, "bf16", [256] * 6),
    # fewer items than compute units: the workspace runs each item as P equal pieces (fan split)
    ("fan split, long prefix", 2, 128, 8000, 300, 1, 300, "bf16", [300, 300]),
    ("fan split, causal blocks", 3, 128, 4000, 700, 1, 100, "bf16", [700, 700]),
    ("fan split, fp32", 2, 64, 3000, 200, 1, 200, "f32", [200, 200]),
]


@pytest.mark.parametrize("schedule", ["split", "whole"])
@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_degenerate_and_ragged_shapes(sr, case, schedule):
    name, H, D, P, cap, W, cb, dtype, chunks = case
    say(f"[edge] {name} ({schedule})")
    _stream_vs_oracle(sr, H, D, P, cap, W, cb, dtype, 31, chunks, SCHEDULES[schedule])


# Queue split with more items than compute units, not a multiple of the 8 XCDs, so that the
# XCDs own different item counts and different numbers of split items (none on some of them);
# causal blocks inside the chunk give the items different tile counts, so split items have
# different piece counts and some levels of the device queue hold empty pieces.
QUEUE_EDGE = [  # H, D, P, cap, W, cb, dtype, chunks
    ("308 items, causal blocks, D=128", 11, 128, 500, 7000, 1, 1000, "bf16", [7000, 7000]),
    ("260 items, half the XCDs without split items, D=64", 20, 64, 0, 3300, 2, 3300, "bf16", [3300] * 3),
    ("260 items, fp32", 20, 64, 0, 3300, 2, 3300, "f32", [3300] * 3),
]


@pytest.mark.parametrize("case", QUEUE_EDGE, ids=[c[0] for c in QUEUE_EDGE])
def test_queue_split_uneven_xcds(sr, case):
    name, H, D, P, cap, W, cb, dtype, chunks = case
    say(f"[queue edge] {name}")
    _stream_vs_oracle(sr, H, D, P, cap, W, cb, dtype, 33, chunks, "own")


@pytest.mark.parametrize("schedule", ["split", "whole"])
def test_most_visible_pages(sr, schedule):
    """A call visiting exactly SR_MAX_VISIBLE_PAGES pages (1023 persistent + 1 current) runs and
    matches the oracle on sampled rows; one page more is refused before anything is enqueued."""
    import torch
    P = (sr.MAX_VISIBLE_PAGES - 1) * 128
    say(f"[max pages] P={P} ({schedule})")
    _stream_vs_oracle(sr, 1, 64, P, 256, 0, 256, "bf16", 32, [128], SCHEDULES[schedule],
                      rows=np.array([0, 1, 63, 64, 127]))
    cfg = sr.config_for(1, 64, P, 256, 0, 256, 1, sr.SR_BF16)
    pk = torch.zeros((1, P, 1, 64), dtype=torch.bfloat16, device="cuda")
    cache = sr.KVCache(cfg, pk, pk, workspace=SCHEDULES[schedule])
    x = torch.zeros((129, 1, 64), dtype=torch.bfloat16, device="cuda")
    cache.append(0, x, x)
    with pytest.raises(sr.SrError) as e:
        cache.attention(0, x)
    assert e.value.status == 5  # SR_E_UNSUPPORTED
    cache.close()


def test_state_errors_on_device_cache(sr):
    """Rejected calls enqueue nothing and leave the cache usable and unchanged."""
    import torch
    w = synth.get_workload("t_stream")
    cache, mk, _, _ = _one_chunk_cache(sr, 2, 128, 64, 128, 1, 128, "bf16", 4)
    k, v, q = mk(128, 2, 128), mk(128, 2, 128), mk(128, 2, 128)
    with pytest.raises(sr.SrError) as e:
        cache.attention(0, q)
    assert e.value.status == 2
    cache.append(0, k, v)
    cache.append(1, k, v)
    before = cache.attention(0, q).clone()
    for args, st in [((2, k, v), 2), ((5, k, v), 1)]:
        with pytest.raises(sr.SrError) as e:
            cache.append(*args)
        assert e.value.status == st
    with pytest.raises(sr.SrError) as e:
        cache.attention(1, q)
    assert e.value.status == 1
    assert torch.equal(cache.attention(0, q), before)
    cache.close()
