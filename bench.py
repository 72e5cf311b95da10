"""Benchmark of the streaming chunk-attention hot path on one MI355X.

One step = one streaming chunk-step of one attention layer at full window: evict the
oldest history chunk, append the next chunk's K/V into its ring slot, run chunk attention
of its queries over bank + history + current (StreamRender-H3 project page, "2.3 A
Real-Time Interaction Loop", step 4, and "3.3 Inference Acceleration and End-to-End
Deployment").  Steps cycle over several independent layer caches, the way a DiT forward
visits its layers, so each step finds its cache cold in the 256 MB last-level cache
(the 832x480 workload's K/V are ~200 MB per layer); `--layers 1` gives the warm number.

`--workload c1w` times the page-literal window variant instead: per step, evict, rewrite the
W history chunks in place, append the current chunk, and the attention of all moving rows
(history + current) over the whole window ("3.1.2 Historical Context and Temporal
Consistency", prefix cache).

`--workload c1x` runs the c1 chunk-steps on a reduced-precision cache (MXFP6 keys and
queries, FP8 values: "The road to the fastest, cheapest H3", Accelerating the denoiser,
item 2); its roofline peak is the MFMA peak of that mix (below).

`--workload d1` (or d1s, the shifted layer) times one layer of the streaming decoder at 720p
("3.2 Fast Causal H3 VAE"): per step, evict, rewrite the five global tokens, append the chunk
window by window, every window's attention in one launch and the global tokens' attention.

`--workload c1p` runs c1 chunk-steps whose chunk enters through the fused append
(sr_kvcache_append_qkv: qk-RMSNorm, rotary embedding at stream-absolute positions and the
cache write in one kernel, "3.2 Fast Causal H3 VAE", iteration 6) and reports that kernel's
HBM roofline beside the attention one.

Prints one JSON line (see --help).  Inputs are seeded synthetic tensors resident in HBM
before the timed region; timing brackets exactly --steps steps with device syncs, and HIP
events around each attention launch give the kernel's average duration for the roofline.

    python bench.py [--gpus 1] [--steps 30] [--warmup 5] [--workload c1] [--layers 4]
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 flop/clk x 2.4 GHz, dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # dense fp32 MFMA
PEAK_HBM_GBS = 8000.0
# Reduced-precision attention: half of the algorithmic flops (Q.K^T) run on the FP6 matrix
# rate (10.1 PFLOP/s dense), half (P.V) on the FP8 rate (5.0 PFLOP/s); the time at peak is
# F/2 / 10.1 + F/2 / 5.0, i.e. an effective peak of 2 / (1/10.1 + 1/5.0) PFLOP/s.
PEAK_MX_TFLOPS = round(2.0 / (1.0 / 10100.0 + 1.0 / 5000.0), 1)
# Reduced-precision workloads: the cache type SR_MX on another workload's shapes and inputs.
MX_WORKLOADS = {"c1x": "c1"}

# Bytes moved past L2 per attention launch, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this
# script (profiles/chunk_attention_<workload>_counters.md), scaled by the factors a plain
# 256 MiB device copy gives in the same runs (fetched = 2.0 x FETCH_SIZE, written = 1.0 x
# WRITE_SIZE).  Each entry holds the SHA-256 of the attention kernel source it was measured
# on; the figure is reported only while that source is unchanged.
TRAFFIC = {
    "c1": {"fetch_kib": 327292.3, "write_kib": 92316.6,
           "attention_sha256": "bb1ab0dc1a53ce62094c5886dacc69e54838bc79bec8f7fefea6d55f9146c6e0"},
    "c3": {"fetch_kib": 1234596.9, "write_kib": 139502.6,
           "attention_sha256": "bb1ab0dc1a53ce62094c5886dacc69e54838bc79bec8f7fefea6d55f9146c6e0"},
    "c1w": {"fetch_kib": 344903.0, "write_kib": 109618.2,
            "attention_sha256": "bb1ab0dc1a53ce62094c5886dacc69e54838bc79bec8f7fefea6d55f9146c6e0"},
    "c1x": {"fetch_kib": 179635.4, "write_kib": 125190.2,
            "attention_sha256": "bb1ab0dc1a53ce62094c5886dacc69e54838bc79bec8f7fefea6d55f9146c6e0"},
    # the decoder layer's dominant kernel: windows_attention_kernel
    "d1": {"fetch_kib": 115315.1, "write_kib": 31079.7,
           "attention_sha256": "bb1ab0dc1a53ce62094c5886dacc69e54838bc79bec8f7fefea6d55f9146c6e0"},
}
ATTENTION_SRC = os.path.join(ROOT, "chunk_causal_attention_amd", "csrc", "attention.hip")
# The same counts for the fused-append kernel (prep_append_kernel in kv_kernels.hip), per launch.
PREP_TRAFFIC = {
    "c1p": {"fetch_kib": 42327.2, "write_kib": 84912.0,
            "kv_sha256": "fa43d4c0a4050000aba2dd574b944cc817eb06ccaf5f22b74b50a422f45d25b6"},
}
KV_SRC = os.path.join(ROOT, "chunk_causal_attention_amd", "csrc", "kv_kernels.hip")


def attention_source_sha256():
    import hashlib
    with open(ATTENTION_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload):
    """Scaled bytes per launch for `workload`, or None if not measured on this kernel source."""
    t = TRAFFIC.get(workload)
    if not t or t["fetch_kib"] is None or t["attention_sha256"] != attention_source_sha256():
        return None
    return (2.0 * t["fetch_kib"] + 1.0 * t["write_kib"]) * 1024.0


def measured_prep_traffic(workload):
    """Scaled bytes per fused-append launch, or None if not measured on this kernel source."""
    import hashlib
    t = PREP_TRAFFIC.get(workload)
    if not t or t["kv_sha256"] != hashlib.sha256(open(KV_SRC, "rb").read()).hexdigest():
        return None
    return (2.0 * t["fetch_kib"] + 1.0 * t["write_kib"]) * 1024.0


def attention_flops(w):
    """Algorithmic flops of one call: 4 * H * D * sum_i |S(i)| (visible pairs only)."""
    n, cb = w.chunk, w.causal_block
    fixed = w.persistent + w.window * w.chunk
    i = np.arange(n)
    vis = fixed + np.minimum(n, (i // cb + 1) * cb)
    return 4.0 * w.heads * w.head_dim * float(vis.sum())


def append_bytes(w, mx=False):
    """Algorithmic bytes of one append: read K,V [n][H][D] + write their pages (the slot's zero
    tail included); reduced-precision pages hold 25 bytes per 32 K features (padded to whole KiB
    per page) and one byte per V feature."""
    es = 2 if w.dtype == "bf16" else 4
    pages = math.ceil(w.chunk / 128)
    if mx:
        kpage = (w.head_dim // 32 * 3200 + 1023) // 1024 * 1024
        return es * w.heads * w.head_dim * 2 * w.chunk + w.heads * pages * (kpage + 128 * w.head_dim)
    return es * w.heads * w.head_dim * 2 * (w.chunk + pages * 128)


def _native_cache(w, pk, pv, hist, cur, conv=None):
    """The C++ oracle's cache holding the workload's last chunk-step (conv maps storage values)."""
    from oracle import native
    conv = conv or (lambda a: a)
    m = native.StreamingCache(conv(pk), conv(pv), w.window)
    for i, (k, v) in enumerate(hist):
        m.append(i, conv(k), conv(v))
    m.append(len(hist), conv(cur[0]), conv(cur[1]))
    return m


def _timed_heads(w, run, budget_s, group):
    """Runs run(heads) on groups of heads until every head is done or budget_s has passed."""
    done, t0 = 0, time.perf_counter()
    while done < w.heads and time.perf_counter() - t0 < budget_s:
        hs = list(range(done, min(w.heads, done + group)))
        run(hs)
        done += len(hs)
    return done, time.perf_counter() - t0


def cpu_baseline(w, budget_s=20.0):
    """The plain C++ fp64 oracle, as it stands, on whole heads of the workload's last chunk-step,
    with every hardware thread (std::thread over head x 64-row blocks)."""
    import synth
    from oracle import native
    pk, pv, hist, cur = synth.single_step_inputs(w)
    m = _native_cache(w, pk, pv, hist, cur)
    scale = 1.0 / math.sqrt(w.head_dim)
    threads = native.load().orc_hardware_threads()
    heads, dt = _timed_heads(w, lambda hs: native.chunk_attention(m, 0, cur[2], scale, w.causal_block, w.dtype,
                                                                  heads=hs), budget_s, 4)
    flops = attention_flops(w) * heads / w.heads
    model, _ = native.cpu_model()
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": model,
            "sample": f"{heads} of {w.heads} heads x all {w.chunk} query rows of {w.name} "
                      f"({w.visible_keys} keys), C++ fp64 oracle on {threads} threads, {dt:.1f} s wall"}


def cpu_baseline_mx(w, budget_s=20.0):
    """The C++ oracle on whole heads of the reduced-precision chunk-step: the heads' queries, keys
    and values quantized by oracle.mx (MXFP6 q/k, FP8 v; exact in fp32), then the fp64 attention
    over the dequantized values.  The quantization is timed with the attention."""
    import oracle
    import synth
    from oracle import mx as omx
    from oracle import native
    pk, pv, hist, cur = synth.single_step_inputs(w)
    wid = lambda a: oracle.widen(a, "bf16")
    scale = 1.0 / math.sqrt(w.head_dim)
    threads = native.load().orc_hardware_threads()

    def run(hs):
        h = slice(hs[0], hs[-1] + 1)
        dk = lambda a: omx.mxfp6_values(wid(a[..., h, :])).astype(np.float32)
        dv = lambda a: omx.fp8_values(wid(a[..., h, :])).astype(np.float32)
        m = native.StreamingCache(dk(pk), dv(pv), w.window)
        for i, (k, v) in enumerate(hist):
            m.append(i, dk(k), dv(v))
        m.append(len(hist), dk(cur[0]), dv(cur[1]))
        native.chunk_attention(m, 0, dk(cur[2]), scale, w.causal_block, "f32")

    heads, dt = _timed_heads(w, run, budget_s, 4)
    flops = attention_flops(w) * heads / w.heads
    model, _ = native.cpu_model()
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": model,
            "sample": f"{heads} of {w.heads} heads x all {w.chunk} query rows of {w.name} ({w.visible_keys} keys): "
                      f"MXFP6/FP8 quantization of those heads' inputs (numpy) + fp64 attention over the "
                      f"dequantized values (C++ oracle, {threads} threads), {dt:.1f} s wall"}


def make_inputs(sr, w, n_sets, torch):
    """Device-resident chunk inputs (K, V, Q) and the persistent bank, from the seeded generator."""
    import synth
    from synth.torch_io import to_dev
    stream = synth.SessionStream(w)
    pk, pv = stream.persistent()
    sets = []
    for ev in stream:
        sets.append(tuple(to_dev(ev[x], w.dtype) for x in ("k", "v", "q")))
        if len(sets) == n_sets:
            break
    return to_dev(pk, w.dtype), to_dev(pv, w.dtype), sets


def copy_calibration(res, torch, dev):
    """A plain device copy of known size, for scaling the profiler's HBM byte counters, and the same
    bytes read once with the attention kernel's global-to-LDS page loads (sr_probe_lds_read), which
    shows that one factor serves both."""
    import chunk_causal_attention_amd as sr
    n = 256 << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    sink = torch.empty(n // 256, dtype=torch.float32, device=dev)
    for _ in range(3):
        dst.copy_(src)
        sr.sr_probe_lds_read(src, sink)
    torch.cuda.synchronize()
    res["copy_calibration_bytes"] = n


# Workloads run in the page-literal window variant (moving rows over the whole window).
WINDOW_WORKLOADS = ("c1w",)


def window_flops(w):
    """Algorithmic flops of one window call: every moving row sees every key of the window."""
    m = (w.window + 1) * w.chunk
    return 4.0 * w.heads * w.head_dim * m * float(w.persistent + m)


def cpu_baseline_window(w, budget_s=10.0):
    """The fp64 oracle, as it stands, on whole heads of the window variant's full-window step."""
    import oracle
    import synth
    from threadpoolctl import threadpool_info
    stream = synth.WindowStream(w)
    pk, pv = stream.persistent()
    m = oracle.StreamingCache(pk, pv, w.window)
    ev = None
    for ev in stream:
        if ev["evict_before"]:
            m.evict()
        for i, k, v in ev["history"]:
            m.update(i, k, v)
        m.append(ev["chunk"], ev["k"], ev["v"])
    scale = 1.0 / math.sqrt(w.head_dim)
    heads, t0 = 0, time.perf_counter()
    while heads < w.heads and time.perf_counter() - t0 < budget_s:
        oracle.window_attention(m, ev["bank"], ev["q"], scale, w.dtype, heads=[heads])
        heads += 1
    dt = time.perf_counter() - t0
    flops = window_flops(w) * heads / w.heads
    threads = max([x.get("num_threads", 1) for x in threadpool_info()] + [1])
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{heads} of {w.heads} heads x all {ev['q'].shape[0]} moving rows of {w.name} "
                      f"({w.persistent + ev['q'].shape[0]} keys), fp64 numpy oracle, {dt:.1f} s wall"}


def run_window(args, w):
    """Window-variant step: evict, rewrite the W history chunks in place, append the current
    chunk, and the moving rows' attention over the whole window."""
    import torch
    import synth
    import chunk_causal_attention_amd as sr
    from synth.torch_io import to_dev

    torch.cuda.init()
    dev = torch.device("cuda:0")
    stream = synth.WindowStream(w)
    pk, pv = (to_dev(x, w.dtype) for x in stream.persistent())
    full = None
    for ev in stream:
        full = ev          # the last chunk-step: full window
    hist = [(to_dev(k, w.dtype), to_dev(v, w.dtype)) for _, k, v in full["history"]]
    kc, vc, q = (to_dev(full[x], w.dtype) for x in ("k", "v", "q"))
    scale = 1.0 / math.sqrt(w.head_dim)
    cfg = sr.config_for(w.heads, w.head_dim, w.persistent, w.chunk, w.window, w.causal_block, w.banks,
                        sr.SR_BF16 if w.dtype == "bf16" else sr.SR_F32)
    t_init = time.perf_counter()
    layers = []
    ws = None if args.no_split else sr.workspace_for(cfg)
    for _ in range(args.layers):
        c = sr.KVCache(cfg, pk, pv, workspace=ws)
        for j in range(w.window + 1):
            c.append(j, kc, vc)
        layers.append({"cache": c, "next": w.window + 1})
    torch.cuda.synchronize()
    t_init = time.perf_counter() - t_init
    m = q.shape[0]
    out = torch.empty_like(q)
    lse = torch.empty((w.heads, m), dtype=torch.float32, device=dev)
    ev_pairs = []

    def step(i, timed):
        L = layers[i % len(layers)]
        c = L["cache"]
        cid = L["next"]
        L["next"] += 1
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)] if timed else None
        if w.window > 0:
            c.evict()
        if timed:
            e[0].record()
        for j, (k, v) in enumerate(hist):
            c.update(cid - w.window + j, k, v)
        c.append(cid, kc, vc)
        if timed:
            e[1].record()
        c.window_attention(cid % w.banks, q, out=out, lse=lse, softmax_scale=scale)
        if timed:
            e[2].record()
            ev_pairs.append(e)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    t_write = np.array([a.elapsed_time(b) for a, b, _ in ev_pairs])
    t_attn = np.array([b.elapsed_time(c) for _, b, c in ev_pairs])
    ms_step = elapsed * 1e3 / args.steps
    F = window_flops(w)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    attn_tflops = F / (t_attn.mean() * 1e-3) / 1e12
    traffic = (measured_traffic(w.name) if w == synth.get_workload(w.name) else None)
    if args.traffic_kib is not None:
        traffic = args.traffic_kib * 1024.0
    res = {
        "metric": "ms per window step & attention TFLOP/s (frac of bf16 MFMA peak), 1 MI355X",
        "value": round(F / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: window step (page-literal variant), {w.heads} heads x {w.head_dim}, "
                        f"{m} moving rows ({w.window}x{w.chunk} history + {w.chunk} current) over "
                        f"{w.persistent} persistent + {m} window tokens, bidirectional",
            "heads": w.heads, "head_dim": w.head_dim, "queries": m, "keys_visible": w.persistent + m,
            "layers_cycled": args.layers,
            "step": "evict + update_chunk x W + append_chunk + window_attention",
            "schedule": "whole items" if args.no_split else "key tiles split evenly over the CUs",
            "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(attn_tflops, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / peak, 4),
            "traffic": traffic,
        },
        "ms_attention": round(float(t_attn.mean()), 4),
        "ms_attention_p10_p50_p90": [round(float(np.percentile(t_attn, p)), 4) for p in (10, 50, 90)],
        "ms_kv_writes": round(float(t_write.mean()), 4),
        "kv_writes_GBps": round((w.window + 1) * append_bytes(w) / (t_write.mean() * 1e-3) / 1e9, 1),
        "attention_gflop_per_call": round(F / 1e9, 3),
        "session_init_ms_per_layer": round(t_init * 1e3 / args.layers, 3),
    }
    for L in layers:
        L["cache"].close()
    if args.copy_calibration:
        copy_calibration(res, torch, dev)
    if args.cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_window(w, args.cpu_budget)
    return res


# Workloads whose chunks enter through the fused append (qk-RMSNorm + rotary + cache write).
PREP_WORKLOADS = ("c1p",)
PEAK_HBM_GBPS = 8000.0
# Latent grid of the 832x480 workloads: 52 x 30 tokens per latent frame.
GRID_W, FRAME_TOKENS = 52, 1560


def prep_bytes(w):
    """Algorithmic bytes of one fused append: read qkv [n][3][H][D] and the positions; write the
    prepared queries [n][H][D] and the K/V pages of the slot (with its zero tail)."""
    es = 2 if w.dtype == "bf16" else 4
    slot_tokens = math.ceil(w.chunk / 128) * 128
    return es * w.heads * w.head_dim * (3 * w.chunk + w.chunk + 2 * slot_tokens) + 12 * w.chunk


def run_prep(args, w):
    """Fused-append step: evict, append the chunk's qkv projection through the fused kernel
    (queries and keys RMS-normalised and rotated at their stream-absolute positions), then
    chunk attention of the prepared queries."""
    import torch
    import synth
    import chunk_causal_attention_amd as sr
    from synth.torch_io import to_dev

    torch.cuda.init()
    dev = torch.device("cuda:0")
    pk, pv = (to_dev(x, w.dtype) for x in synth.SessionStream(w).persistent())
    n_sets = w.window + 2
    qkvs = [to_dev(synth.qkv_inputs(w, w.chunk, chunk=j), w.dtype) for j in range(n_sets)]
    frames = w.chunk // FRAME_TOKENS
    poss = [torch.from_numpy(synth.latent_positions(w.chunk, FRAME_TOKENS, GRID_W, frames * j)).to(dev)
            for j in range(n_sets)]
    gq, gk = (torch.from_numpy(g).to(dev) for g in synth.prep_gains(w))
    prep = sr.qk_prep((w.head_dim // 8, 3 * w.head_dim // 16, 3 * w.head_dim // 16), 10000.0, 1e-6)
    scale = 1.0 / math.sqrt(w.head_dim)
    cfg = sr.config_for(w.heads, w.head_dim, w.persistent, w.chunk, w.window, w.causal_block, w.banks,
                        sr.SR_BF16 if w.dtype == "bf16" else sr.SR_F32)
    q = torch.empty((w.chunk, w.heads, w.head_dim), dtype=qkvs[0].dtype, device=dev)
    t_init = time.perf_counter()
    layers = []
    ws = None if args.no_split else sr.workspace_for(cfg)
    for _ in range(args.layers):
        c = sr.KVCache(cfg, pk, pv, workspace=ws)
        for j in range(w.window + 1):
            c.append_qkv(j, qkvs[j % n_sets], poss[j % n_sets], gq, gk, prep, q_out=q)
        layers.append({"cache": c, "next": w.window + 1})
    torch.cuda.synchronize()
    t_init = time.perf_counter() - t_init
    out = torch.empty_like(q)
    lse = torch.empty((w.heads, w.chunk), dtype=torch.float32, device=dev)
    ev_pairs = []

    def step(i, timed):
        L = layers[i % len(layers)]
        c = L["cache"]
        cid = L["next"]
        L["next"] += 1
        if w.window > 0:
            c.evict()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)] if timed else None
        if timed:
            e[0].record()
        c.append_qkv(cid, qkvs[cid % n_sets], poss[cid % n_sets], gq, gk, prep, q_out=q)
        if timed:
            e[1].record()
        c.attention(cid % w.banks, q, out=out, lse=lse, softmax_scale=scale)
        if timed:
            e[2].record()
            ev_pairs.append(e)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    t_prep = np.array([a.elapsed_time(b) for a, b, _ in ev_pairs])
    t_attn = np.array([b.elapsed_time(c) for _, b, c in ev_pairs])
    ms_step = elapsed * 1e3 / args.steps
    F = attention_flops(w)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    attn_tflops = F / (t_attn.mean() * 1e-3) / 1e12
    prep_gbps = prep_bytes(w) / (t_prep.mean() * 1e-3) / 1e9
    res = {
        "metric": "ms per chunk-step & attention TFLOP/s (frac of bf16 MFMA peak), 1 MI355X",
        "value": round(F / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: chunk-step through the fused append, {w.heads} heads x {w.head_dim}, "
                        f"{w.persistent} persistent + {w.window}x{w.chunk} history + {w.chunk} current tokens",
            "heads": w.heads, "head_dim": w.head_dim, "queries": w.chunk, "keys_visible": w.visible_keys,
            "layers_cycled": args.layers,
            "step": "evict + append_qkv (qk-RMSNorm + rotary + cache write) + chunk_attention",
            "schedule": "whole items" if args.no_split else "key tiles split evenly over the CUs",
            "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(attn_tflops, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / peak, 4),
            "traffic": (measured_traffic(w.name) if w == synth.get_workload(w.name) else None),
        },
        "prep_roofline": {
            "bound": "hbm",
            "achieved": round(prep_gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(prep_gbps / PEAK_HBM_GBPS, 4),
            "traffic": (measured_prep_traffic(w.name) if w == synth.get_workload(w.name) else None),
        },
        "ms_attention": round(float(t_attn.mean()), 4),
        "ms_attention_p10_p50_p90": [round(float(np.percentile(t_attn, p)), 4) for p in (10, 50, 90)],
        "ms_append_qkv": round(float(t_prep.mean()), 4),
        "ms_append_qkv_p10_p50_p90": [round(float(np.percentile(t_prep, p)), 4) for p in (10, 50, 90)],
        "append_qkv_bytes": prep_bytes(w),
        "attention_gflop_per_call": round(F / 1e9, 3),
        "session_init_ms_per_layer": round(t_init * 1e3 / args.layers, 3),
    }
    for L in layers:
        L["cache"].close()
    if args.copy_calibration:
        copy_calibration(res, torch, dev)
    if args.cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    return res


# Decoder layers: the streaming decoder's window attention ("3.2 Fast Causal H3 VAE").
DECODER_WORKLOADS = ("d1", "d1s")


def decoder_flops(w):
    """Algorithmic flops of one decoder layer's attention at full ring: every window's rows over
    the global tokens and the window's tokens of W + 1 chunks, and the global tokens over the
    global tokens and the whole chunk.  Returns (windows, global)."""
    r = w.frames * np.asarray(w.window_tokens, dtype=np.float64)
    f_win = 4.0 * w.heads * w.head_dim * float((r * (w.global_tokens + (w.window_chunks + 1) * r)).sum())
    f_glob = 4.0 * w.heads * w.head_dim * w.global_tokens * float(w.global_tokens + w.chunk_tokens)
    return f_win, f_glob


def global_bytes(w):
    """Algorithmic bytes of one global-token call: the K/V of the global tokens and of every frame
    token of the chunk, read once; the queries read and the outputs written once."""
    es = 2 if w.dtype == "bf16" else 4
    G = w.global_tokens
    return es * w.heads * w.head_dim * (2 * (G + w.chunk_tokens) + 2 * G)


# Bytes past L2 per launch of the few-row split-K kernel (few_attention_kernel), as TRAFFIC.
FEW_TRAFFIC = {
    "d1": {"fetch_kib": 30209.5, "write_kib": 684.9,
           "few_sha256": "d8e1fecb5cf618f8d94159acbf7b53df3c0f5337c9f65ef3d0e297511606532d"},
}
FEW_SRC = os.path.join(ROOT, "chunk_causal_attention_amd", "csrc", "few_attention.hip")


def measured_few_traffic(workload):
    import hashlib
    t = FEW_TRAFFIC.get(workload)
    if not t or t["few_sha256"] != hashlib.sha256(open(FEW_SRC, "rb").read()).hexdigest():
        return None
    return (2.0 * t["fetch_kib"] + 1.0 * t["write_kib"]) * 1024.0


def cpu_baseline_decoder(w, budget_s=10.0):
    """The fp64 oracle, as it stands, on whole heads of the decoder layer's full-ring chunk."""
    import oracle
    import synth
    from threadpoolctl import threadpool_info
    z = np.zeros((1, w.global_tokens, w.heads, w.head_dim), dtype=np.uint16)
    m = oracle.StreamingCache(z, z, w.window_chunks)
    ev = None
    for ev in synth.DecoderStream(w):
        if ev["evict_before"]:
            m.evict()
        m.set_bank(0, ev["gk"], ev["gv"])
        m.append(ev["chunk"], ev["k"], ev["v"])
    scale = 1.0 / math.sqrt(w.head_dim)
    heads, t0 = 0, time.perf_counter()
    while heads < w.heads and time.perf_counter() - t0 < budget_s:
        oracle.decoder_window_attention(m, w.window_tokens, w.frames, ev["q"], scale, w.dtype, heads=[heads])
        oracle.decoder_global_attention(m, ev["gq"], scale, w.dtype, heads=[heads])
        heads += 1
    dt = time.perf_counter() - t0
    flops = sum(decoder_flops(w)) * heads / w.heads
    threads = max([x.get("num_threads", 1) for x in threadpool_info()] + [1])
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{heads} of {w.heads} heads of {w.name}: every window's rows and the global rows of the "
                      f"full-ring chunk, fp64 numpy oracle, {dt:.1f} s wall"}


def run_decoder(args, w):
    """Decoder-layer step: evict the oldest chunk, rewrite the global tokens, append the chunk
    window by window, every window's attention (one launch) and the global tokens' attention."""
    import torch
    import synth
    import chunk_causal_attention_amd as sr
    from synth.torch_io import to_dev

    torch.cuda.init()
    dev = torch.device("cuda:0")
    evs = list(synth.DecoderStream(w))
    sets = [tuple(to_dev(ev[x], w.dtype) for x in ("gk", "gv", "k", "v", "q", "gq")) for ev in evs]
    scale = 1.0 / math.sqrt(w.head_dim)
    G, T = w.global_tokens, w.chunk_tokens
    cfg = sr.config_for(w.heads, w.head_dim, G, w.capacity, w.window_chunks, w.capacity, 1,
                        sr.SR_BF16 if w.dtype == "bf16" else sr.SR_F32)
    zero = torch.zeros((1, G, w.heads, w.head_dim), dtype=sets[0][0].dtype, device=dev)
    t_init = time.perf_counter()
    layers = []
    ws = None if args.no_split else sr.workspace_for(cfg)
    for _ in range(args.layers):
        c = sr.KVCache(cfg, zero, zero, workspace=ws)
        c.set_window_layout(w.window_tokens, w.frames, w.window_pages)
        for j in range(w.window_chunks + 1):
            gk, gv, k, v, _, _ = sets[j % len(sets)]
            c.set_bank(0, gk, gv)
            c.append_windows(j, k, v)
        layers.append({"cache": c, "next": w.window_chunks + 1})
    torch.cuda.synchronize()
    t_init = time.perf_counter() - t_init
    out = torch.empty((T, w.heads, w.head_dim), dtype=zero.dtype, device=dev)
    lse = torch.empty((w.heads, T), dtype=torch.float32, device=dev)
    gout = torch.empty((G, w.heads, w.head_dim), dtype=zero.dtype, device=dev)
    glse = torch.empty((w.heads, G), dtype=torch.float32, device=dev)
    ev_sets = []

    def step(i, timed):
        L = layers[i % len(layers)]
        c = L["cache"]
        cid = L["next"]
        L["next"] += 1
        gk, gv, k, v, q, gq = sets[cid % len(sets)]
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if timed else None
        if w.window_chunks > 0:
            c.evict()
        if timed:
            e[0].record()
        c.set_bank(0, gk, gv)
        c.append_windows(cid, k, v)
        if timed:
            e[1].record()
        c.windows_attention(0, q, out=out, lse=lse, softmax_scale=scale)
        if timed:
            e[2].record()
        c.global_attention(0, gq, out=gout, lse=glse, softmax_scale=scale)
        if timed:
            e[3].record()
            ev_sets.append(e)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    t_write = np.array([e[0].elapsed_time(e[1]) for e in ev_sets])
    t_win = np.array([e[1].elapsed_time(e[2]) for e in ev_sets])
    t_glob = np.array([e[2].elapsed_time(e[3]) for e in ev_sets])
    ms_step = elapsed * 1e3 / args.steps
    f_win, f_glob = decoder_flops(w)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    win_tflops = f_win / (t_win.mean() * 1e-3) / 1e12
    glob_gbps = global_bytes(w) / (t_glob.mean() * 1e-3) / 1e9
    stock = w == synth.get_decoder_workload(w.name)   # counters were taken on the stock shapes
    traffic = measured_traffic(w.name) if stock else None
    if args.traffic_kib is not None:
        traffic = args.traffic_kib * 1024.0
    es = 2 if w.dtype == "bf16" else 4
    # K and V read once, their pages (zero tails included) written once: the bank's, then every window's.
    write_bytes = es * w.heads * w.head_dim * 2 * (G + 128 * math.ceil(G / 128) + T + w.capacity)
    rmax = w.frames * max(w.window_tokens)
    res = {
        "metric": "decoder-layer attention TFLOP/s per chunk (frac of bf16 MFMA peak), 1 MI355X",
        "value": round((f_win + f_glob) / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: decoder layer at {w.grid_h}x{w.grid_w} latent tokens, {len(w.window_tokens)} "
                        f"windows of {w.window}x{w.window} tokens (offset {w.shift}), {w.frames} frames per chunk, "
                        f"{w.window_chunks} cached chunks, {G} global tokens, {w.heads} heads x {w.head_dim}",
            "heads": w.heads, "head_dim": w.head_dim, "windows": len(w.window_tokens), "queries_per_chunk": T,
            "largest_window": f"{rmax} queries x {G + (w.window_chunks + 1) * rmax} keys",
            "layers_cycled": args.layers,
            "step": "evict + set_bank + append_windows + windows_attention + global_attention",
            "global_schedule": "whole items" if args.no_split else "key tiles split evenly over the CUs",
            "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(win_tflops, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(win_tflops / peak, 4),
            "traffic": traffic,
        },
        "global_roofline": {
            "bound": "hbm",
            "achieved": round(glob_gbps, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(glob_gbps / PEAK_HBM_GBS, 4),
            "traffic": measured_few_traffic(w.name) if stock else None,
        },
        "ms_windows_attention": round(float(t_win.mean()), 4),
        "ms_windows_attention_p10_p50_p90": [round(float(np.percentile(t_win, p)), 4) for p in (10, 50, 90)],
        "ms_global_attention": round(float(t_glob.mean()), 4),
        "global_attention_TFLOPs": round(f_glob / (t_glob.mean() * 1e-3) / 1e12, 3),
        "ms_kv_writes": round(float(t_write.mean()), 4),
        "kv_writes_GBps": round(write_bytes / (t_write.mean() * 1e-3) / 1e9, 1),
        "windows_gflop_per_call": round(f_win / 1e9, 3),
        "global_gflop_per_call": round(f_glob / 1e9, 4),
        "session_init_ms_per_layer": round(t_init * 1e3 / args.layers, 3),
    }
    for L in layers:
        L["cache"].close()
    if args.copy_calibration:
        copy_calibration(res, torch, dev)
    if args.cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decoder(w, args.cpu_budget)
    return res


def time_chunk_steps(sr, torch, w, mx, n_layers, steps, warmup, no_split):
    """Cold chunk-steps of workload w: n_layers independent layer caches (each larger than the
    last-level cache for the full-size workloads) visited in turn, every step evict + append +
    chunk attention, HIP events on the launch stream around the append and the attention."""
    dev = torch.device("cuda:0")
    pk, pv, sets = make_inputs(sr, w, w.window + 2, torch)
    scale = 1.0 / math.sqrt(w.head_dim)
    cfg = sr.config_for(w.heads, w.head_dim, w.persistent, w.chunk, w.window, w.causal_block, w.banks,
                        sr.SR_MX if mx else (sr.SR_BF16 if w.dtype == "bf16" else sr.SR_F32))
    t_init = time.perf_counter()
    layers = []
    # One attention workspace serves every layer cache: their calls are ordered on one stream.
    ws = None if no_split else sr.workspace_for(cfg)
    for _ in range(n_layers):
        c = sr.KVCache(cfg, pk, pv, workspace=ws)
        for j in range(w.window + 1):
            k, v, _ = sets[j % len(sets)]
            c.append(j, k, v)
        layers.append({"cache": c, "next": w.window + 1})
    torch.cuda.synchronize()
    t_init = time.perf_counter() - t_init
    out = torch.empty((w.chunk, w.heads, w.head_dim), dtype=sets[0][0].dtype, device=dev)
    lse = torch.empty((w.heads, w.chunk), dtype=torch.float32, device=dev)
    ev_pairs = []

    def step(i, timed):
        L = layers[i % len(layers)]
        c = L["cache"]
        cid = L["next"]
        L["next"] += 1
        if w.window > 0:
            c.evict()
        k, v, q = sets[cid % len(sets)]
        if timed:
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            e0.record()
            c.append(cid, k, v)
            e1.record()
            c.attention(cid % w.banks, q, out=out, lse=lse, softmax_scale=scale)
            e2.record()
            ev_pairs.append((e0, e1, e2))
        else:
            c.append(cid, k, v)
            c.attention(cid % w.banks, q, out=out, lse=lse, softmax_scale=scale)

    for i in range(warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    res = {"elapsed": elapsed, "init_s": t_init,
           "append_ms": np.array([a.elapsed_time(b) for a, b, _ in ev_pairs]),
           "attention_ms": np.array([b.elapsed_time(c) for _, b, c in ev_pairs])}
    for L in layers:
        L["cache"].close()
    del layers, out, lse, sets
    torch.cuda.empty_cache()
    return res


def mfma_probe(sr, torch, dev, iters=8000, reps=5):
    """The dense bf16 MFMA rate the device sustains (sr_probe_mfma_bf16: two workgroups of eight
    waves per compute unit, four independent MFMA chains per wave, register operands), best of
    `reps` launches, and the shader clock it implies at 4096 flop per clock and compute unit."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = 2 * cus
    out = torch.empty(wgs * 512, dtype=torch.float32, device=dev)
    flops = wgs * 8 * 4 * 32768.0 * iters
    sr.sr_probe_mfma_bf16(out, wgs, 100)
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        sr.sr_probe_mfma_bf16(out, wgs, iters)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None or ms < best else best
    tf = flops / (best * 1e-3) / 1e12
    return {"tflops": round(tf, 1), "frac_of_spec": round(tf / PEAK_BF16_TFLOPS, 4),
            "clock_mhz_implied": round(tf * 1e12 / (cus * 4096.0) / 1e6, 0), "ms": round(best, 4),
            "method": f"{wgs} workgroups x 8 waves x 4 MFMA chains x {iters} v_mfma_f32_32x32x16_bf16, best of {reps}"}


def run(args):
    import torch
    import synth
    import chunk_causal_attention_amd as sr

    sr.load()
    if args.workload in DECODER_WORKLOADS:
        w = synth.get_decoder_workload(args.workload)
        if args.window_chunks is not None:
            w = w.scaled(window_chunks=args.window_chunks, chunks=args.window_chunks + 2)
        return run_decoder(args, w)
    mx = args.workload in MX_WORKLOADS
    w = synth.get_workload(MX_WORKLOADS.get(args.workload, args.workload))
    if args.heads is not None:
        # one GPU's share of a run whose heads are sharded over several GPUs (same shapes, fewer heads)
        w = w.scaled(heads=args.heads)
    if w.name in WINDOW_WORKLOADS:
        return run_window(args, w)
    if w.name in PREP_WORKLOADS:
        return run_prep(args, w)
    if not w.single_step:
        raise SystemExit(f"workload {w.name} is a parity case, not a bench workload")
    torch.cuda.init()
    dev = torch.device("cuda:0")
    t = time_chunk_steps(sr, torch, w, mx, args.layers, args.steps, args.warmup, args.no_split)
    elapsed, t_append, t_attn, t_init = t["elapsed"], t["append_ms"], t["attention_ms"], t["init_s"]
    ms_step = elapsed * 1e3 / args.steps
    F = attention_flops(w)
    peak = PEAK_MX_TFLOPS if mx else (PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS)
    attn_tflops = F / (t_attn.mean() * 1e-3) / 1e12
    name = args.workload
    traffic = measured_traffic(name) if args.heads is None else None
    if args.traffic_kib is not None:
        traffic = args.traffic_kib * 1024.0
    res = {
        "metric": "ms per chunk-step & attention TFLOP/s (frac of bf16 MFMA peak), 1 MI355X" if not mx else
                  "ms per chunk-step & attention TFLOP/s (frac of the FP6/FP8 MFMA peak), 1 MI355X",
        "value": round(F / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp6 q.k, fp8 p.v" if mx else w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{name}: chunk-step, {w.heads} heads x {w.head_dim}, {w.persistent} persistent + "
                        f"{w.window}x{w.chunk} history + {w.chunk} current tokens, causal block {w.causal_block}"
                        + (", reduced-precision cache (MXFP6 keys/queries, FP8 values)" if mx else ""),
            "heads": w.heads, "head_dim": w.head_dim, "queries": w.chunk, "keys_visible": w.visible_keys,
            "layers_cycled": args.layers, "step": "evict + append_chunk + chunk_attention",
            "schedule": "whole items" if args.no_split else "key tiles split evenly over the CUs",
            "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(attn_tflops, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / peak, 4),
            "traffic": traffic,
        },
        "ms_attention": round(float(t_attn.mean()), 4),
        "ms_attention_p10_p50_p90": [round(float(np.percentile(t_attn, p)), 4) for p in (10, 50, 90)],
        "ms_append": round(float(t_append.mean()), 4),
        "append_GBps": round(append_bytes(w, mx) / (t_append.mean() * 1e-3) / 1e9, 1),
        "attention_gflop_per_call": round(F / 1e9, 3),
        "session_init_ms_per_layer": round(t_init * 1e3 / args.layers, 3),
    }
    if name == "c1" and args.heads is None and not args.no_split and args.extra_c3:
        # the second configuration of the target, timed the same way (cold, split schedule)
        w3 = synth.get_workload("c3")
        t3 = time_chunk_steps(sr, torch, w3, False, args.layers, max(10, args.steps // 2), args.warmup, False)
        a3 = t3["attention_ms"]
        tf3 = attention_flops(w3) / (a3.mean() * 1e-3) / 1e12
        res["c3_ms_attention"] = round(float(a3.mean()), 4)
        res["c3_ms_attention_p10_p50_p90"] = [round(float(np.percentile(a3, p)), 4) for p in (10, 50, 90)]
        res["c3_attention_tflops"] = round(tf3, 3)
        res["c3_frac"] = round(tf3 / PEAK_BF16_TFLOPS, 4)
        res["c3_steps"] = len(a3)
    if args.probe and not mx and w.dtype == "bf16":
        probe = mfma_probe(sr, torch, dev)
        probe["attention_frac_of_probe"] = round(attn_tflops / probe["tflops"], 4)
        if "c3_attention_tflops" in res:
            probe["c3_frac_of_probe"] = round(res["c3_attention_tflops"] / probe["tflops"], 4)
        res["mfma_probe"] = probe
    if args.copy_calibration:
        copy_calibration(res, torch, dev)
    if args.cpu_baseline:
        res["cpu_baseline"] = (cpu_baseline_mx if mx else cpu_baseline)(w, args.cpu_budget)
    return res


# Counter passes of --counters: one rocprofv3 run each (a run may hold at most 8 SQ, 4 TCC,
# 2 GRBM counters; FETCH_SIZE takes 3 TCC, WRITE_SIZE 2).
COUNTER_PASSES = [
    ("fetch", ["FETCH_SIZE"]),
    ("write", ["WRITE_SIZE"]),
    ("mfma", ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES",
              "SQ_VALU_MFMA_COEXEC_CYCLES", "GRBM_GUI_ACTIVE", "GRBM_COUNT"]),
    ("mix", ["SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_MFMA", "SQ_INSTS_SALU",
             "SQ_INSTS_LDS", "SQ_INSTS_VMEM"]),
    ("lds", ["SQ_WAIT_INST_LDS", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT",
             "SQ_LDS_IDX_ACTIVE", "SQ_LDS_CMD_FIFO_FULL"]),
    ("l2", ["TCC_HIT_sum", "TCC_MISS_sum"]),
]
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def dominant_kernel(workload):
    """Name fragment of the kernel the roofline is about for `workload`."""
    return "windows_attention_kernel" if workload in DECODER_WORKLOADS else "chunk_attention_kernel"


def attention_bytes(w):
    """Algorithmic bytes of one chunk-attention call: Q and O once, the K and V of every visible key
    once (bf16 / fp32 caches)."""
    es = 2 if w.dtype == "bf16" else 4
    return es * w.heads * w.head_dim * (2.0 * w.chunk + 2.0 * w.visible_keys)


def _counter_means(csv_path, fragment):
    """Mean per dispatch of every counter of the kernels whose name contains `fragment`, and the
    mean dispatch duration (ns)."""
    import csv
    vals, durs = {}, {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if fragment not in r["Kernel_Name"]:
                continue
            vals.setdefault(r["Counter_Name"], {})[r["Dispatch_Id"]] = float(r["Counter_Value"])
            durs[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    means = {k: sum(v.values()) / len(v) for k, v in vals.items()}
    return means, (sum(durs.values()) / len(durs) if durs else None), len(durs)


def run_counters(args):
    """Every pass of COUNTER_PASSES as its own rocprofv3 run of this script (a child process, under a
    hard time limit), on the workload's default launch with the 256 MiB copy calibration; returns
    the per-dispatch means of the dominant kernel and the derived figures."""
    import signal
    import subprocess
    import synth
    out_dir = os.path.abspath(args.counters_dir)
    os.makedirs(out_dir, exist_ok=True)
    child = [sys.executable, "-u", os.path.abspath(__file__), "--workload", args.workload, "--no-cpu-baseline",
             "--no-extra-c3", "--no-probe", "--steps", "4", "--warmup", "2", "--layers", str(args.layers),
             "--copy-calibration"]
    if args.no_split:
        child.append("--no-split")
    env = dict(os.environ, TMPDIR="/tmp")
    frag = args.counters_kernel or dominant_kernel(args.workload)
    raw, dur, calib, cmds = {}, None, {}, []
    for name, ctrs in COUNTER_PASSES:
        cmd = ["rocprofv3", "--pmc"] + ctrs + ["--output-format", "csv", "-d", os.path.join(out_dir, name),
                                               "-o", name, "--"] + child
        cmds.append(" ".join(cmd))
        print(f"[counters] pass {name}: {' '.join(ctrs)}", file=sys.stderr, flush=True)
        p = subprocess.Popen(cmd, cwd="/tmp", env=env, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE,
                             start_new_session=True)
        try:
            _, err = p.communicate(timeout=args.counters_timeout)
        except subprocess.TimeoutExpired:
            os.killpg(p.pid, signal.SIGKILL)
            p.wait()
            raise SystemExit(f"counter pass {name} exceeded {args.counters_timeout} s")
        csv_path = os.path.join(out_dir, name, f"{name}_counter_collection.csv")
        if not os.path.exists(csv_path):
            raise SystemExit(f"counter pass {name} failed (exit {p.returncode}): {err.decode()[-2000:]}")
        means, d, n = _counter_means(csv_path, frag)
        raw.update(means)
        dur = d if dur is None else dur
        if name in ("fetch", "write"):
            cm, _, _ = _counter_means(csv_path, COPY_KERNEL)
            calib.update(cm)
        if name == "fetch":
            lm, _, _ = _counter_means(csv_path, "lds_read_probe_kernel")
            calib["LDS_FETCH_SIZE"] = lm.get("FETCH_SIZE")
    copy_bytes = 256 << 20
    fetch_factor = copy_bytes / (calib["FETCH_SIZE"] * 1024.0)   # about 2: FETCH_SIZE counts half of each request
    write_factor = copy_bytes / (calib["WRITE_SIZE"] * 1024.0)
    fetched = fetch_factor * raw["FETCH_SIZE"] * 1024.0
    written = write_factor * raw["WRITE_SIZE"] * 1024.0
    xcds = 8
    gui = raw.get("GRBM_GUI_ACTIVE", 0.0) / xcds
    res = {
        "workload": args.workload, "kernel": frag, "dispatches_per_pass": n,
        "mean_dispatch_us_under_counters": round(dur / 1e3, 2) if dur else None,
        "counters": {k: round(v, 1) for k, v in sorted(raw.items())},
        "copy_calibration": {"fetch_factor": round(fetch_factor, 3), "write_factor": round(write_factor, 3),
                             "lds_read_fetch_factor": (round(copy_bytes / (calib["LDS_FETCH_SIZE"] * 1024.0), 3)
                                                       if calib.get("LDS_FETCH_SIZE") else None)},
        "fetch_kib": round(raw["FETCH_SIZE"], 1), "write_kib": round(raw["WRITE_SIZE"], 1),
        "traffic_bytes": round(fetched + written),
        "attention_sha256": attention_source_sha256(),
        "commands": cmds,
    }
    if frag == dominant_kernel(args.workload) and args.workload not in DECODER_WORKLOADS + ("c1w",) \
            and args.workload not in MX_WORKLOADS:
        w = synth.get_workload(args.workload)
        res["algorithmic_bytes"] = round(attention_bytes(w))
        res["traffic_ratio"] = round((fetched + written) / attention_bytes(w), 3)
    if gui > 0 and dur:
        res["clock_ghz_from_gui_active"] = round(gui / dur, 3)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in raw:
            res["mfma_busy_frac"] = round(raw["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * 1024.0), 4)
    if raw.get("SQ_INSTS_MFMA"):
        res["valu_per_mfma"] = round(raw["SQ_INSTS_VALU"] / raw["SQ_INSTS_MFMA"], 3)
        res["lds_insts_per_mfma"] = round(raw.get("SQ_INSTS_LDS", 0.0) / raw["SQ_INSTS_MFMA"], 3)
    if raw.get("SQ_WAVE_CYCLES"):
        res["wait_any_frac"] = round(raw.get("SQ_WAIT_ANY", 0.0) / raw["SQ_WAVE_CYCLES"], 4)
    if raw.get("TCC_HIT_sum") is not None and raw.get("TCC_MISS_sum") is not None:
        res["l2_hit_frac"] = round(raw["TCC_HIT_sum"] / max(raw["TCC_HIT_sum"] + raw["TCC_MISS_sum"], 1.0), 4)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="c1",
                    help="c1 (default), c3, c4, c1s, c4s; c1w: the page-literal window variant at c1 shapes; "
                         "c1p: c1 chunk-steps entering through the fused qk-RMSNorm + rotary append; "
                         "c1x: c1 chunk-steps on the reduced-precision (MXFP6/FP8) cache; "
                         "d1, d1s: a 720p streaming-decoder layer (plain or shifted windows)")
    ap.add_argument("--layers", type=int, default=4, help="independent layer caches cycled over")
    ap.add_argument("--heads", type=int, default=None,
                    help="chunk workloads: heads of one GPU's share of a head-sharded run (e.g. 3 = 24 over 8)")
    ap.add_argument("--window-chunks", type=int, default=None,
                    help="decoder workloads: cached chunks W (default: the workload's, 2 = four latent frames)")
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--no-split", action="store_true",
                    help="run attention without a workspace (one workgroup per head and query tile)")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work (whole heads)")
    ap.add_argument("--no-extra-c3", dest="extra_c3", action="store_false",
                    help="c1: do not also time the 720p workload c3's attention (reported as c3_* keys)")
    ap.add_argument("--no-probe", dest="probe", action="store_false",
                    help="do not run the dense bf16 MFMA probe (reported as mfma_probe)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB device copy (reference for the profiler's byte counters)")
    ap.add_argument("--traffic-kib", type=float, default=None,
                    help="override: scaled KiB per attention launch from rocprofv3 FETCH/WRITE runs")
    ap.add_argument("--counters", action="store_true",
                    help="instead of timing: run rocprofv3 counter passes of this workload (traffic, MFMA busy, "
                         "instruction mix, LDS, L2) as child runs and print their per-dispatch means as JSON")
    ap.add_argument("--counters-dir", default="gpurun_out/counters", help="--counters: where rocprofv3 writes")
    ap.add_argument("--counters-timeout", type=float, default=240.0, help="--counters: seconds per pass")
    ap.add_argument("--counters-kernel", default=None,
                    help="--counters: name fragment of the kernel to report (default: the workload's attention kernel)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU: the multi-GPU path is not implemented",
                          "n_gpus": args.gpus}))
        raise SystemExit(2)
    res = run_counters(args) if args.counters else run(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
