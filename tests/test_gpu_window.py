"""GPU parity of the page-literal window variant against the fp64 oracle.

sr_window_attention (the moving rows -- history chunks and the current chunk -- over the
whole window, bidirectionally), sr_prefix_attention (a bank's prefix rows over that bank)
and sr_kvcache_update_chunk (history chunks rewritten in place every step), called through
the C ABI.  Element by element on reduced streams and at the c1 window shape.
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


SCHEDULES = {"split": "own", "whole": None}


def _stats(out_h, lse_h, o_ref, l_ref, dtype, rows):
    return (gates.error_stats(harness.widen_host(out_h[rows], dtype), o_ref),
            gates.error_stats(lse_h[:, rows], l_ref))


def run_window_stream(sr, w, rows=None, workspace="own", check_gather=False, prefix_rows=None):
    """Streams workload `w` in the page-literal variant through the library and the oracle
    model: every step rewrites the history chunks in place, appends the current chunk and
    runs the moving rows' attention; each bank's prefix rows run once at the start."""
    import torch
    scale = 1.0 / np.sqrt(w.head_dim)
    stream = synth.WindowStream(w)
    pk, pv = stream.persistent()
    cache = sr.KVCache(harness.cfg_of(sr, w), harness.to_dev(pk, w.dtype), harness.to_dev(pv, w.dtype),
                       workspace=workspace)
    model = oracle.StreamingCache(pk, pv, w.window)
    stats = []
    for b in range(w.banks):
        qp = stream.prefix_queries(b)
        lse = torch.empty((w.heads, w.persistent), dtype=torch.float32, device="cuda")
        out = cache.prefix_attention(b, harness.to_dev(qp, w.dtype), lse=lse, softmax_scale=scale)
        r = np.arange(w.persistent) if prefix_rows is None else prefix_rows
        o_ref, l_ref = oracle.prefix_attention(model, b, qp, scale, w.dtype, rows=r)
        out_h = harness.to_host(out, w.dtype)
        assert np.isfinite(harness.widen_host(out_h, w.dtype)).all()
        stats.append((("prefix", b),) + _stats(out_h, lse.cpu().numpy(), o_ref, l_ref, w.dtype, r))
    for idx, ev in enumerate(stream):
        c = ev["chunk"]
        if ev["evict_before"]:
            assert cache.evict() == model.evict()
        for i, k, v in ev["history"]:
            cache.update(i, harness.to_dev(k, w.dtype), harness.to_dev(v, w.dtype))
            model.update(i, k, v)
        cache.append(c, harness.to_dev(ev["k"], w.dtype), harness.to_dev(ev["v"], w.dtype))
        model.append(c, ev["k"], ev["v"])
        if w.single_step and c != w.chunks - 1:
            continue
        q = ev["q"]
        lse = torch.empty((w.heads, q.shape[0]), dtype=torch.float32, device="cuda")
        out = cache.window_attention(ev["bank"], harness.to_dev(q, w.dtype), lse=lse, softmax_scale=scale)
        if check_gather:
            kg, vg = cache.gather(ev["bank"])
            km, vm, _ = model.sequence(ev["bank"])
            assert (harness.to_host(kg, w.dtype) == km).all() and (harness.to_host(vg, w.dtype) == vm).all(), \
                (w.name, idx)
        out_h = harness.to_host(out, w.dtype)
        assert np.isfinite(harness.widen_host(out_h, w.dtype)).all()
        r = np.arange(q.shape[0]) if rows is None else rows[rows < q.shape[0]]
        o_ref, l_ref = oracle.window_attention(model, ev["bank"], q, scale, w.dtype, rows=r)
        stats.append((("window", idx),) + _stats(out_h, lse.cpu().numpy(), o_ref, l_ref, w.dtype, r))
    cache.close()
    return stats


def check_stats(w, stats):
    g = gates.gates_for(w.dtype)
    lse_tol = 2e-2 if w.dtype == "bf16" else 1e-4
    for what, st, st_l in stats:
        assert gates.passes(st, g), (w.name, what, st)
        assert st_l["max_abs"] <= lse_tol, (w.name, what, st_l)


@pytest.mark.parametrize("schedule", ["split", "whole"])
@pytest.mark.parametrize("name", ["t_win", "t_win64", "t_winf32"])
def test_window_parity_every_element(sr, name, schedule):
    w = synth.get_workload(name)
    say(f"[window] {name} ({schedule}): H={w.heads} D={w.head_dim} P={w.persistent} chunk={w.chunk} W={w.window}")
    stats = run_window_stream(sr, w, workspace=SCHEDULES[schedule], check_gather=True)
    assert len(stats) == w.banks + w.chunks * w.steps
    check_stats(w, stats)
    say(f"[window] {name}: worst", max(s[1]["max_abs"] for s in stats), max(s[1]["rel_fro"] for s in stats))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("schedule", ["split", "whole"])
def test_window_full_size(sr, schedule):
    """c1 window shape: 3 x 4680 moving rows over 2072 + 14040 keys, 24 heads, and the prefix
    rows' call over the 2072-token bank.  Every element in the benchmark's launch configuration
    (split schedule; with 1320 items the planner runs them whole anyway); sampled rows with no
    workspace."""
    w = synth.get_workload("c1w")
    if schedule == "split":
        rows = prow = None
        say(f"[window full] c1w ({schedule}): every moving and prefix row")
    else:
        rows = harness.sample_rows(w.chunk * (w.window + 1))
        prow = harness.sample_rows(w.persistent)
        say(f"[window full] c1w ({schedule}): {len(rows)} sampled moving rows, {len(prow)} prefix rows")
    stats = run_window_stream(sr, w, rows=rows, prefix_rows=prow, workspace=SCHEDULES[schedule])
    check_stats(w, stats)
    say("[window full] c1w:", stats[-1][1], "lse", stats[-1][2]["max_abs"])


def test_window_without_history_equals_chunk_attention(sr):
    """With no history and causal_block >= chunk, the moving rows are the current chunk and
    every row sees the whole window either way: the two calls give the same bits."""
    import torch
    rng = np.random.default_rng(3)
    H, D, P, n = 3, 128, 200, 500
    cfg = sr.config_for(H, D, P, n, 2, n, 1, sr.SR_BF16)
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s).astype(np.float32)).to(torch.bfloat16).cuda()
    cache = sr.KVCache(cfg, mk(1, P, H, D), mk(1, P, H, D))
    cache.append(7, mk(n, H, D), mk(n, H, D))
    q = mk(n, H, D)
    l1 = torch.empty((H, n), dtype=torch.float32, device="cuda")
    l2 = torch.empty_like(l1)
    o1 = cache.attention(0, q, lse=l1)
    o2 = cache.window_attention(0, q, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    cache.close()


def test_window_call_errors(sr):
    """Rejected window/prefix/update calls enqueue nothing and leave the cache unchanged."""
    import torch
    rng = np.random.default_rng(5)
    H, D, P, n = 2, 128, 64, 128
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s).astype(np.float32)).to(torch.bfloat16).cuda()
    cache = sr.KVCache(sr.config_for(H, D, P, n, 1, n, 1, sr.SR_BF16), mk(1, P, H, D), mk(1, P, H, D))
    k, v = mk(n, H, D), mk(n, H, D)
    with pytest.raises(sr.SrError) as e:
        cache.window_attention(0, mk(n, H, D))
    assert e.value.status == 2                      # no current chunk yet
    qp = mk(P, H, D)
    op = cache.prefix_attention(0, qp).clone()      # needs no current chunk
    cache.append(0, k, v)
    cache.append(1, k, v)
    before = cache.window_attention(0, mk(2 * n, H, D) * 0 + 1).clone()
    for rows in (n, 2 * n - 1, 2 * n + 1):
        with pytest.raises(sr.SrError) as e:
            cache.window_attention(0, mk(rows, H, D))
        assert e.value.status == 1
    for cid in (2, -1, 5):
        with pytest.raises(sr.SrError) as e:
            cache.update(cid, k, v)
        assert e.value.status == 1
    with pytest.raises(sr.SrError) as e:
        cache.update(0, mk(n + 1, H, D), mk(n + 1, H, D))   # longer than the slot
    assert e.value.status == 1
    assert torch.equal(cache.window_attention(0, mk(2 * n, H, D) * 0 + 1), before)
    assert torch.equal(cache.prefix_attention(0, qp), op)
    cache.evict()
    with pytest.raises(sr.SrError) as e:
        cache.update(0, k, v)                       # evicted
    assert e.value.status == 1
    cache.close()
    empty = sr.KVCache(sr.config_for(H, D, 0, n, 1, n, 1, sr.SR_BF16))
    with pytest.raises(sr.SrError) as e:
        empty.prefix_attention(0, mk(1, H, D))
    assert e.value.status == 1                      # no persistent tokens
    empty.close()
