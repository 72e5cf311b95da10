"""The no-allocation global-token attention (sr_global_attention_static) through the C ABI.

Its records and counters live in the library's static scratch instead of the cache's
workspace; otherwise it is the same split-K call as sr_global_attention with a workspace
attached, so the two must agree bit for bit, and both must match the oracle.  Two calls in a
row, the second with a smaller input (fewer heads, pages and rows), the second one checked for
allocating nothing; a call that needs more scratch than the array holds is refused.
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


def _last_chunk_cache(sr, w):
    """A windowed cache (with a workspace) and the oracle's model, streamed to the last chunk."""
    cfg = sr.config_for(w.heads, w.head_dim, w.global_tokens, w.capacity, w.window_chunks, w.capacity, 1, sr.SR_BF16)
    z = np.zeros((1, w.global_tokens, w.heads, w.head_dim), dtype=np.uint16)
    cache = sr.KVCache(cfg, harness.to_dev(z, "bf16"), harness.to_dev(z, "bf16"), workspace="own")
    cache.set_window_layout(w.window_tokens, w.frames, w.window_pages)
    model = oracle.StreamingCache(z, z, w.window_chunks)
    last = None
    for ev in synth.DecoderStream(w):
        if ev["evict_before"]:
            assert cache.evict() == model.evict()
        cache.set_bank(0, harness.to_dev(ev["gk"], "bf16"), harness.to_dev(ev["gv"], "bf16"))
        model.set_bank(0, ev["gk"], ev["gv"])
        cache.append_windows(ev["chunk"], harness.to_dev(ev["k"], "bf16"), harness.to_dev(ev["v"], "bf16"))
        model.append(ev["chunk"], ev["k"], ev["v"])
        last = ev
    return cache, model, last


def _check_call(sr, w, rows, check_alloc):
    import torch
    scale = 1.0 / np.sqrt(w.head_dim)
    cache, model, ev = _last_chunk_cache(sr, w)
    gq = ev["gq"][:rows]
    q = harness.to_dev(np.ascontiguousarray(gq), "bf16")
    out_ws = torch.empty((rows, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    lse_ws = torch.empty((w.heads, rows), dtype=torch.float32, device="cuda")
    out_st = torch.full_like(out_ws, float("nan"))
    lse_st = torch.full_like(lse_ws, float("nan"))
    cache.global_attention(0, q, out=out_ws, lse=lse_ws, softmax_scale=scale)
    torch.cuda.synchronize()
    before = (torch.cuda.memory_allocated(), torch.cuda.mem_get_info()[0])
    cache.global_attention_static(0, q, out=out_st, lse=lse_st, softmax_scale=scale)
    torch.cuda.synchronize()
    after = (torch.cuda.memory_allocated(), torch.cuda.mem_get_info()[0])
    if check_alloc:
        assert before == after, (before, after)
    assert torch.equal(out_st, out_ws) and torch.equal(lse_st, lse_ws)
    g_ref, gl_ref = oracle.decoder_global_attention(model, gq, scale, "bf16")
    st = gates.error_stats(harness.widen_host(harness.to_host(out_st, "bf16"), "bf16"), g_ref)
    st_l = gates.error_stats(lse_st.cpu().numpy(), gl_ref)
    assert gates.passes(st, gates.gates_for("bf16")), st
    assert st_l["max_abs"] <= 2e-2, st_l
    cache.close()
    return st


def test_static_scratch_global_attention_two_calls(sr):
    """d1 (16 heads, 5 rows over 5 + 7200 keys), then a smaller call (t_dec: 3 heads, 3 rows)."""
    say("[no-alloc] d1, 5 global rows")
    st1 = _check_call(sr, synth.get_decoder_workload("d1"), 5, check_alloc=False)
    say("[no-alloc] t_dec, 3 global rows (smaller)")
    st2 = _check_call(sr, synth.get_decoder_workload("t_dec"), 3, check_alloc=True)
    say(f"[no-alloc] max-abs {st1['max_abs']:.3g}, {st2['max_abs']:.3g}")


def test_static_scratch_refuses_oversize_calls(sr):
    """64 heads x 5 pieces (17 pages, four per piece) x (64 + 32 x 128) floats of records exceed
    the 2^20-float array: the call is refused before anything is enqueued and the output stays
    untouched."""
    import torch
    H, D, G, cap = 64, 128, 5, 16 * 128
    cfg = sr.config_for(H, D, G, cap, 1, cap, 1, sr.SR_BF16)
    z = torch.zeros((1, G, H, D), dtype=torch.bfloat16, device="cuda")
    cache = sr.KVCache(cfg, z, z, workspace="own")
    cache.set_window_layout([1024], 2, 16)
    x = torch.zeros((2048, H, D), dtype=torch.bfloat16, device="cuda")
    cache.append_windows(0, x, x)
    q = torch.zeros((32, H, D), dtype=torch.bfloat16, device="cuda")
    out = torch.full((32, H, D), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sr.SrError) as e:
        cache.global_attention_static(0, q, out=out)
    assert e.value.status == 5  # SR_E_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    small = cache.global_attention_static(0, q[:4])  # 64 x 5 x (64 + 4 x 128) floats fit
    torch.cuda.synchronize()
    assert torch.isfinite(small.float()).all()
    cache.close()
