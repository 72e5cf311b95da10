"""GPU parity of the fused append (sr_kvcache_append_qkv: qk-RMSNorm, rotary embedding and the
cache write after the qkv projection) against the fp64 oracle.

The prepared queries and keys are compared element by element with oracle.prep_qkv: the
kernel computes in fp32 and rounds once to the storage type, so every element must lie
within that rounding (bf16: 2^-8 relative) plus the fp32 arithmetic before it (see
_ulp_check).  Values pass through bit for bit.  A stream of chunks appended
this way and attended with the prepared queries must match the oracle's pipeline within the
attention gates.
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


def _sections(D):
    return (D // 8, 3 * D // 16, 3 * D // 16)     # 128 -> (16, 24, 24); 64 -> (8, 12, 12)


def _ulp_check(dev, ref, dtype, what):
    """|dev - ref| within the final rounding to the storage type (bf16: half an ulp, at most
    2^-8 |ref|) plus the fp32 arithmetic before it: the mean square of up to 128 terms
    (relative error below 4e-6) and the rotation, whose error is absolute in the pair's size
    (about 2^-23 x |pair| <= 1e-6 here) when its two products nearly cancel."""
    rel = 2.0 ** -8 if dtype == "bf16" else 4e-6
    err = np.abs(dev - ref)
    bound = rel * np.abs(ref) + 2e-6
    bad = err > bound
    assert not bad.any(), (what, int(bad.sum()), float(err.max()), float((err / np.maximum(np.abs(ref), 1e-30)).max()))
    return float(err.max())


@pytest.mark.parametrize("dtype,D,n,first_frame", [("bf16", 128, 333, 5000), ("bf16", 64, 200, 7),
                                                    ("f32", 64, 150, 123456)])
def test_prep_every_element(sr, dtype, D, n, first_frame):
    import torch
    H, P, cap = 3, 70, 400
    w = synth.get_workload("t_stream").scaled(heads=H, head_dim=D, dtype=dtype)
    say(f"[prep] {dtype} D={D} n={n} first frame {first_frame}")
    qkv = synth.qkv_inputs(w, n, chunk=1)
    pos = synth.latent_positions(n, 60, 10, first_frame)
    gq, gk = synth.prep_gains(w)
    sec = _sections(D)
    cfg = sr.config_for(H, D, P, cap, 1, cap, 1, sr.SR_BF16 if dtype == "bf16" else sr.SR_F32)
    pk = harness.to_dev(np.zeros((1, P, H, D), np.uint16 if dtype == "bf16" else np.float32), dtype)
    cache = sr.KVCache(cfg, pk, pk)
    dq = cache.append_qkv(4, harness.to_dev(qkv, dtype), torch.from_numpy(pos).cuda(), torch.from_numpy(gq).cuda(),
                          torch.from_numpy(gk).cuda(), sr.qk_prep(sec, 10000.0, 1e-6))
    kg, vg = cache.gather(0)
    torch.cuda.synchronize()
    q_ref, k_ref, _ = oracle.prep_qkv(qkv, pos, gq.astype(np.float64), gk.astype(np.float64), 1e-6, sec, 10000.0,
                                      dtype)
    eq = _ulp_check(harness.widen_host(harness.to_host(dq, dtype), dtype), q_ref, dtype, "q")
    ek = _ulp_check(harness.widen_host(harness.to_host(kg, dtype), dtype)[P:], k_ref, dtype, "k")
    assert (harness.to_host(vg, dtype)[P:] == qkv[:, 2]).all()
    assert kg.shape[0] == P + n
    say(f"[prep] max |err| q {eq:.3g} k {ek:.3g}")
    cache.close()


def test_prep_full_size_every_element(sr):
    """The benchmark's c1p call: a 4680-token chunk (three 52 x 30 latent frames from stream frame
    300 on) x 24 heads x 128 into a c1 cache, rotation sections 16/24/24, base 10^4, eps 10^-6;
    every element of the prepared q and k against the oracle, V bit for bit."""
    import torch
    w = synth.get_workload("c1p")
    n, H, D = w.chunk, w.heads, w.head_dim
    say(f"[prep full] c1p: {n} tokens x {H} heads x {D}")
    qkv = synth.qkv_inputs(w, n, chunk=100)
    pos = synth.latent_positions(n, 1560, 52, 300)
    gq, gk = synth.prep_gains(w)
    sec = _sections(D)
    cfg = harness.cfg_of(sr, w)
    pk, pv = synth.SessionStream(w).persistent()   # storage arrays [1][P][H][D]
    cache = sr.KVCache(cfg, harness.to_dev(pk, w.dtype), harness.to_dev(pv, w.dtype))
    dq = cache.append_qkv(0, harness.to_dev(qkv, w.dtype), torch.from_numpy(pos).cuda(), torch.from_numpy(gq).cuda(),
                          torch.from_numpy(gk).cuda(), sr.qk_prep(sec, 10000.0, 1e-6))
    kg, vg = cache.gather(0)
    torch.cuda.synchronize()
    q_ref, k_ref, _ = oracle.prep_qkv(qkv, pos, gq.astype(np.float64), gk.astype(np.float64), 1e-6, sec, 10000.0,
                                      w.dtype)
    P = w.persistent
    eq = _ulp_check(harness.widen_host(harness.to_host(dq, w.dtype), w.dtype), q_ref, w.dtype, "q")
    ek = _ulp_check(harness.widen_host(harness.to_host(kg, w.dtype), w.dtype)[P:], k_ref, w.dtype, "k")
    assert (harness.to_host(vg, w.dtype)[P:] == qkv[:, 2]).all()
    assert (harness.to_host(kg, w.dtype)[:P] == pk[0]).all()
    say(f"[prep full] max |err| q {eq:.3g} k {ek:.3g}")
    cache.close()


def test_prep_stream_attention(sr):
    """Chunks appended with the fused call, then chunk attention of the prepared queries:
    the oracle runs the same pipeline (prep_qkv, its cache model, chunk_attention) in fp64."""
    import torch
    w = synth.get_workload("t_stream").scaled(ar_rho=0.0)
    H, D, P, n, W = w.heads, w.head_dim, w.persistent, w.chunk, w.window
    sec = _sections(D)
    prep = sr.qk_prep(sec, 10000.0, 1e-6)
    gq, gk = synth.prep_gains(w)
    stream = synth.SessionStream(w)
    pk, pv = stream.persistent()
    cache = sr.KVCache(harness.cfg_of(sr, w), harness.to_dev(pk, "bf16"), harness.to_dev(pv, "bf16"))
    f32 = lambda a: oracle.widen(a, "bf16").astype(np.float32)
    model = oracle.StreamingCache(f32(pk), f32(pv), W)
    scale = 1.0 / np.sqrt(D)
    frames = 2                                  # latent frames per chunk (300 tokens each)
    worst = 0.0
    for c in range(w.chunks):
        if W > 0 and c >= W + 1:
            assert cache.evict() == model.evict()
        for s in range(w.steps):
            qkv = synth.qkv_inputs(w, n, chunk=c, step=s)
            pos = synth.latent_positions(n, n // frames, 20, frames * c)
            dq = cache.append_qkv(c, harness.to_dev(qkv, "bf16"), torch.from_numpy(pos).cuda(),
                                  torch.from_numpy(gq).cuda(), torch.from_numpy(gk).cuda(), prep)
            out = cache.attention(s % w.banks, dq, softmax_scale=scale)
            q_ref, k_ref, v_ref = oracle.prep_qkv(qkv, pos, gq.astype(np.float64), gk.astype(np.float64), 1e-6,
                                                  sec, 10000.0, "bf16")
            model.append(c, k_ref.astype(np.float32), v_ref.astype(np.float32))
            o_ref, _ = oracle.chunk_attention(model, s % w.banks, q_ref.astype(np.float32), scale, w.causal_block,
                                              "f32")
            st = gates.assert_gates(harness.widen_host(harness.to_host(out, "bf16"), "bf16"), o_ref, "bf16",
                                    f"chunk {c} step {s}")
            worst = max(worst, st["max_abs"])
    say(f"[prep stream] {w.chunks} chunks x {w.steps} steps, worst max |err| {worst:.3g}")
    cache.close()


def test_prep_stream_clock(sr):
    """The same latent frames attended from different stream clocks (time positions offset by
    0, 100 and 1000) give the same outputs up to the rounding of the rotated values (project
    page 3.2, iteration 4: scores depend only on time differences)."""
    import torch
    H, D, P, n = 2, 128, 0, 256
    w = synth.get_workload("t_stream").scaled(heads=H, head_dim=D)
    sec = _sections(D)
    gq, gk = synth.prep_gains(w)
    qkv0, qkv1 = synth.qkv_inputs(w, n, chunk=0), synth.qkv_inputs(w, n, chunk=1)
    outs = []
    for offset in (0, 100, 1000):
        cache = sr.KVCache(sr.config_for(H, D, P, n, 1, n, 1, sr.SR_BF16))
        for c, qkv in enumerate((qkv0, qkv1)):
            pos = synth.latent_positions(n, 128, 16, offset + 2 * c)
            dq = cache.append_qkv(c, harness.to_dev(qkv, "bf16"), torch.from_numpy(pos).cuda(),
                                  torch.from_numpy(gq).cuda(), torch.from_numpy(gk).cuda(), sr.qk_prep(sec))
        outs.append(harness.widen_host(harness.to_host(cache.attention(0, dq), "bf16"), "bf16"))
        cache.close()
    for o in outs[1:]:
        st = gates.error_stats(o, outs[0])
        assert st["max_abs"] <= 2e-2 and st["rel_fro"] <= 1e-2, st


def test_prep_call_errors(sr):
    """Bad parameters are refused before anything is enqueued and leave the ring unchanged."""
    import torch
    H, D, n = 2, 64, 100
    cache = sr.KVCache(sr.config_for(H, D, 0, 128, 1, 128, 1, sr.SR_BF16))
    qkv = torch.zeros((n, 3, H, D), dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros((n, 3), dtype=torch.int32, device="cuda")
    g = torch.ones(D, dtype=torch.float32, device="cuda")
    cache.append_qkv(0, qkv, pos, g, g, sr.qk_prep((8, 12, 12)))
    before = cache.segments()
    bad = [sr.qk_prep((8, 12, 11)), sr.qk_prep((-1, 20, 13)), sr.qk_prep((8, 12, 12), base=1.0),
           sr.qk_prep((8, 12, 12), eps=-1.0), sr.qk_prep((8, 12, 12), base=float("inf"))]
    for prep in bad:
        with pytest.raises(sr.SrError) as e:
            cache.append_qkv(1, qkv, pos, g, g, prep)
        assert e.value.status == 1
    with pytest.raises(sr.SrError) as e:                      # q_out overlapping qkv
        cache.append_qkv(1, qkv, pos, g, g, sr.qk_prep((8, 12, 12)), q_out=qkv.view(-1)[:n * H * D].view(n, H, D))
    assert e.value.status == 1
    with pytest.raises(sr.SrError) as e:                      # ring rule: chunk 5 after 0
        cache.append_qkv(5, qkv, pos, g, g, sr.qk_prep((8, 12, 12)))
    assert e.value.status == 1
    assert cache.segments() == before
    cache.close()
