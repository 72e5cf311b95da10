"""The C ABI on the host (no GPU): exports, ring state machine, layout, validation."""
import ctypes
import os
import re

import numpy as np
import pytest

import harness
import oracle

HEADER = os.path.join(harness.ROOT, "include", "sr.h")


@pytest.fixture(scope="module")
def sr():
    return harness.lib_module()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sr_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(sr):
    names = declared_functions()
    assert len(names) >= 15
    lib = sr.load()
    for n in names:
        assert hasattr(lib, n), n


def test_binding_constants_match_header(sr):
    """The binding's constants are the header's #defines."""
    text = open(os.path.join(harness.ROOT, "include", "sr.h")).read()
    defs = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define (SR_\w+) (\d+)", text)}
    assert defs["SR_PAGE_TOKENS"] == sr.PAGE_TOKENS
    assert defs["SR_MAX_WINDOW"] == sr.MAX_WINDOW
    assert defs["SR_MAX_VISIBLE_PAGES"] == sr.MAX_VISIBLE_PAGES
    assert defs["SR_MAX_LAYOUT_WINDOWS"] == sr.MAX_LAYOUT_WINDOWS


def test_window_layout_struct(sr):
    """sr_window_layout as the header declares it: three int32 and SR_MAX_LAYOUT_WINDOWS token
    counts, unused entries zero; the binding refuses more windows than the struct holds."""
    import ctypes
    assert ctypes.sizeof(sr.sr_window_layout) == 4 * (3 + sr.MAX_LAYOUT_WINDOWS)
    lay = sr.window_layout([256] * 10 + [208] * 5, 2, 4)
    assert (lay.num_windows, lay.frames_per_chunk, lay.window_pages) == (15, 2, 4)
    assert list(lay.window_tokens) == [256] * 10 + [208] * 5 + [0] * (sr.MAX_LAYOUT_WINDOWS - 15)
    full = sr.window_layout([1] * sr.MAX_LAYOUT_WINDOWS, 2, 1)
    assert full.num_windows == sr.MAX_LAYOUT_WINDOWS
    with pytest.raises(ValueError):
        sr.window_layout([1] * (sr.MAX_LAYOUT_WINDOWS + 1), 2, 1)


def test_window_layout_check(sr):
    """A layout is refused on the host when a window's tokens of one chunk do not fit its pages
    or exceed the pages one attention call can visit, whatever fits the slot; token counts
    above the int16 range are kept whole (no truncation to a negative count)."""
    cap = 60 * 128  # the decoder's 720p slot: 15 windows x 4 pages
    d1 = sr.config_for(16, 128, 5, cap, 2, cap, 1, sr.SR_BF16)
    sr.sr_window_layout_check(d1, sr.window_layout([256] * 10 + [208] * 5, 2, 4))

    def refused(cfg, lay, status=sr.SR_E_INVALID):
        with pytest.raises(sr.SrError) as e:
            sr.sr_window_layout_check(cfg, lay)
        assert e.value.status == status

    # 40,000 tokens x 4 frames in one window of 1250 pages fits the slot, but it is 1250 pages of
    # keys of a single chunk: more than one call can visit (40,000 would also wrap an int16).
    big = sr.config_for(1, 128, 0, 160000, 0, 160000, 1, sr.SR_BF16)
    refused(big, sr.window_layout([40000], 4, 1250))
    # above the int16 range but within the kernel's reach: accepted whole
    ok = sr.config_for(1, 128, 0, 40064, 0, 40064, 1, sr.SR_BF16)
    sr.sr_window_layout_check(ok, sr.window_layout([40000], 1, 313))
    refused(d1, sr.window_layout([129], 1, 1))          # 129 tokens in one page
    refused(d1, sr.window_layout([65], 2, 1))           # 2 frames x 65 tokens in one page
    refused(d1, sr.window_layout([1] * 16, 2, 4))       # 64 pages of a 60-page slot
    refused(sr.config_for(16, 128, 5, cap, 2, cap, 1, sr.SR_MX), sr.window_layout([256], 2, 4),
            sr.SR_E_UNSUPPORTED)


def test_status_strings(sr):
    assert sr.sr_status_string(0) == "SR_OK"
    assert sr.sr_status_string(2) == "SR_E_STATE"


def _layout_pages(cfg):
    ppb = -(-cfg.persistent_tokens // 128)
    pps = -(-cfg.chunk_capacity // 128)
    return ppb, pps, cfg.num_banks * ppb + (cfg.window_chunks + 1) * pps


@pytest.mark.parametrize("H,D,P,banks,cap,W,dt", [(2, 64, 16, 1, 32, 2, 1), (24, 128, 2072, 1, 4680, 2, 0),
                                                  (40, 128, 4112, 2, 7200, 3, 0), (3, 128, 0, 1, 1, 0, 0)])
def test_required_bytes(sr, H, D, P, banks, cap, W, dt):
    cfg = sr.config_for(H, D, P, cap, W, None, banks, dt)
    _, _, pages = _layout_pages(cfg)
    assert sr.sr_kvcache_required_bytes(cfg) == 2 * H * pages * 128 * D * (2 if dt == 0 else 4)


@pytest.mark.parametrize("H,D,P,banks,cap,W", [(24, 128, 2072, 1, 4680, 2), (3, 64, 130, 1, 333, 1), (2, 128, 0, 1, 1, 0)])
def test_required_bytes_mx(sr, H, D, P, banks, cap, W):
    """SR_MX pool: per (head, page) 3200 * D / 32 bytes of K rounded up to whole KiB, then
    128 * D bytes of V (the layout sr.h documents)."""
    cfg = sr.config_for(H, D, P, cap, W, None, banks, sr.SR_MX)
    _, _, pages = _layout_pages(cfg)
    kpage = -(-(D // 32) * 3200 // 1024) * 1024
    assert sr.sr_kvcache_required_bytes(cfg) == H * pages * (kpage + 128 * D)
    assert kpage == (13312 if D == 128 else 7168)


@pytest.mark.parametrize("H,D,cap,cus", [(24, 128, 4680, 256), (2, 64, 32, 8), (40, 128, 7200, 304), (3, 64, 1, 1)])
def test_attention_workspace_bytes(sr, H, D, cap, cus):
    """Per XCD (C = cus / 8 compute units, at least 1): up to 8 pieces of C split items, one
    record each of 8 waves x 64 lanes x 17 eight-byte words (the output accumulators as bf16 at
    head_dim 128 or fp32 at 64, and the running max and sum), then C int32 arrival counters and
    16 queue counters of the split schedule, padded to 256 bytes."""
    cfg = sr.config_for(H, D, 0, cap, 1)
    C = max(cus // 8, 1)
    assert sr.sr_attention_workspace_bytes(cfg, cus) == 8 * 8 * C * 512 * 17 * 8 + -(-(8 * C + 16) * 4 // 256) * 256


def test_attention_workspace_bytes_validation(sr):
    cfg = sr.config_for(24, 128, 0, 4680, 1)
    with pytest.raises(sr.SrError) as e:
        sr.sr_attention_workspace_bytes(cfg, -1)
    assert e.value.status == 1
    cfg.head_dim = 96
    with pytest.raises(sr.SrError) as e:
        sr.sr_attention_workspace_bytes(cfg, 256)
    assert e.value.status == 5
    lib = sr.load()
    assert lib.sr_attention_workspace_bytes(ctypes.byref(cfg), 256, None) == 1
    assert lib.sr_kvcache_set_workspace(None, None, 0, None) == 1


@pytest.mark.parametrize("field,value,status", [("head_dim", 96, 5), ("head_dim", 0, 5), ("window_chunks", 15, 1),
                                                ("dtype_f32_d128", None, 5),
                                                ("window_chunks", -1, 1), ("num_banks", 0, 1), ("num_heads", 0, 1),
                                                ("chunk_capacity", 0, 1), ("causal_block", 0, 1), ("dtype", 7, 1),
                                                ("persistent_tokens", -3, 1)])
def test_config_validation(sr, field, value, status):
    cfg = sr.config_for(4, 128, 100, 300, 2)
    if field == "dtype_f32_d128":
        cfg.dtype = sr.SR_F32          # fp32 caches support head_dim 64 only
    else:
        setattr(cfg, field, value)
    with pytest.raises(sr.SrError) as e:
        sr.sr_ring_create(cfg)
    assert e.value.status == status
    assert sr.sr_last_error() != ""


def test_init_validation_before_device_work(sr):
    """Bad arguments to sr_kvcache_init fail on the host, without touching a device."""
    lib = sr.load()
    cfg = sr.config_for(2, 64, 16, 32, 2, None, 1, sr.SR_F32)
    need = sr.sr_kvcache_required_bytes(cfg)
    h = ctypes.c_void_p()
    P = ctypes.c_void_p
    cases = [
        (None, need, P(4096), P(4096), 1),          # null pool
        (P(4096 + 16), need, P(4096), P(4096), 1),  # pool not 256-byte aligned
        (P(4096), need - 1, P(4096), P(4096), 3),   # pool too small
        (P(4096), need, None, P(4096), 1),          # persistent K missing with P > 0
        (P(4096), need, P(4100), P(4096), 1),       # persistent K misaligned
    ]
    for pool, nbytes, pk, pv, want in cases:
        st = lib.sr_kvcache_init(ctypes.byref(cfg), pool, nbytes, pk, pv, None, ctypes.byref(h))
        assert st == want, (pool, nbytes, pk, pv, st, sr.sr_last_error())
        assert not h.value
    assert lib.sr_chunk_attention(None, 0, P(4096), P(8192), None, 0.1, None) == 1
    assert lib.sr_window_attention(None, 0, P(4096), 1, P(8192), None, 0.1, None) == 1
    assert lib.sr_prefix_attention(None, 0, P(4096), P(8192), None, 0.1, None) == 1
    assert lib.sr_kvcache_update_chunk(None, 0, P(4096), P(4096), 1, None) == 1
    assert lib.sr_kvcache_append_chunk(None, 0, P(4096), P(4096), 1, None) == 1
    assert lib.sr_kvcache_evict(None, None) == 1
    assert lib.sr_kvcache_destroy(None) == 0


def test_probe_validation_before_device_work(sr):
    """The measurement probes refuse bad arguments on the host, before any launch."""
    lib = sr.load()
    P = ctypes.c_void_p
    assert lib.sr_probe_mfma_bf16(None, 1, 1, None) == 1
    assert lib.sr_probe_mfma_bf16(P(4096), 0, 1, None) == 1
    assert lib.sr_probe_mfma_bf16(P(4096), 1, 0, None) == 1
    assert lib.sr_probe_lds_read(None, 65536, P(4096), None) == 1
    assert lib.sr_probe_lds_read(P(4096), 65536, None, None) == 1
    for nbytes in (0, -65536, 65536 + 16, (1 << 24) * 65536 + 65536):
        assert lib.sr_probe_lds_read(P(4096), nbytes, P(4096), None) == 1, nbytes


def _ring_vs_model(sr, W, P, banks, cap, seed, n_ops=600):
    r = np.random.default_rng(seed)
    cfg = sr.config_for(1, 64, P, cap, W, None, banks, sr.SR_F32)
    ppb, pps, _ = _layout_pages(cfg)
    ring = sr.sr_ring_create(cfg)
    z = np.zeros((1, 1, 1), np.float32)
    pk = np.zeros((banks, P, 1, 1), np.float32)
    model = oracle.StreamingCache(pk, pk, W, capacity=cap)
    lens = {}
    cur = None
    try:
        for _ in range(n_ops):
            op = r.integers(0, 6)
            if op == 5:
                # in-place update of a chunk in the window (or of one that is not)
                ids = model.visible_ids()
                cid = int(r.choice(ids)) if ids and r.random() < 0.8 else int(r.integers(-1, 2100))
                n = int(r.integers(0, cap + 2)) if r.random() < 0.1 else int(r.integers(1, cap + 1))
                try:
                    model.update(cid, np.zeros((n, 1, 1), np.float32), np.zeros((n, 1, 1), np.float32))
                    m_ok = True
                except oracle.CacheStateError:
                    m_ok = False
                try:
                    slot = sr.sr_ring_update(ring, cid, n)
                    r_ok = True
                    assert slot == cid % (W + 1)
                except sr.SrError as ex:
                    r_ok = False
                    assert ex.status == 1
                assert m_ok == r_ok, ("update", cid, n, model.visible_ids())
                if r_ok:
                    lens[cid] = n
            elif op == 0:
                try:
                    e_model = model.evict()
                except oracle.CacheStateError:
                    e_model = None
                try:
                    e_ring = sr.sr_ring_evict(ring)
                except sr.SrError as ex:
                    assert ex.status == 2
                    e_ring = None
                assert e_model == e_ring
            else:
                if cur is None:
                    cid = int(r.integers(0, 2000))
                else:
                    cid = cur + {1: 0, 2: 1, 3: 1, 4: int(r.integers(-2, 3))}[int(op)]
                n = int(r.integers(0, cap + 2)) if r.random() < 0.1 else int(r.integers(1, cap + 1))
                try:
                    model.append(cid, np.zeros((n, 1, 1), np.float32) if n > 0 else z[:0], z[:0] if n == 0 else
                                 np.zeros((n, 1, 1), np.float32))
                    m_ok = True
                except oracle.CacheStateError:
                    m_ok = False
                try:
                    slot, com = sr.sr_ring_append(ring, cid, n)
                    r_ok = True
                    assert slot == cid % (W + 1)
                except sr.SrError as ex:
                    r_ok = False
                    assert ex.status in (1, 2)
                assert m_ok == r_ok, (cid, n, cur, model.visible_ids())
                if r_ok:
                    cur = cid
                    lens[cid] = n
            ids = model.visible_ids()
            if ids:
                for b in range(banks):
                    segs = sr.sr_ring_segments(ring, b)
                    expect = ([(-1, 0, b, b * ppb, P)] if P else []) + \
                             [(i, 1, i % (W + 1), banks * ppb + (i % (W + 1)) * pps, lens[i]) for i in ids[:-1]] + \
                             [(ids[-1], 2, ids[-1] % (W + 1), banks * ppb + (ids[-1] % (W + 1)) * pps, lens[ids[-1]])]
                    assert segs == expect
    finally:
        sr.sr_ring_destroy(ring)


@pytest.mark.parametrize("W,P,banks,cap", [(0, 5, 1, 3), (1, 0, 1, 130), (2, 300, 2, 200), (3, 16, 3, 7),
                                           (14, 1, 1, 1)])
def test_ring_matches_oracle_model(sr, W, P, banks, cap):
    _ring_vs_model(sr, W, P, banks, cap, seed=W * 100 + cap)


def test_ring_errors_leave_state(sr):
    cfg = sr.config_for(1, 128, 10, 50, 2)
    ring = sr.sr_ring_create(cfg)
    with pytest.raises(sr.SrError) as e:
        sr.sr_ring_segments(ring, 0)
    assert e.value.status == 2                       # no current chunk yet
    sr.sr_ring_append(ring, 100, 50)
    sr.sr_ring_append(ring, 101, 20)
    sr.sr_ring_append(ring, 102, 30)
    before = sr.sr_ring_segments(ring, 0)
    for cid, n, st in [(103, 10, 2), (105, 10, 1), (99, 10, 1), (102, 51, 1), (102, 0, 1), (-1, 1, 1)]:
        with pytest.raises(sr.SrError) as e:
            sr.sr_ring_append(ring, cid, n)
        assert e.value.status == st
        assert sr.sr_ring_segments(ring, 0) == before
    with pytest.raises(sr.SrError):
        sr.sr_ring_segments(ring, 1)                 # bank out of range
    assert sr.sr_ring_evict(ring) == 100
    sr.sr_ring_append(ring, 103, 10)
    assert [s[0] for s in sr.sr_ring_segments(ring, 0)] == [-1, 101, 102, 103]
    sr.sr_ring_destroy(ring)


def test_missing_library_fails_loudly(tmp_path):
    """Without libsr.so the binding raises instead of falling back to anything else."""
    import subprocess
    import sys
    code = ("import chunk_causal_attention_amd as m; m.LIB_PATH = %r\n"
            "try:\n    m.load()\nexcept ImportError as e:\n    print('raised', e)\n" % str(tmp_path / "nope.so"))
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=harness.ROOT)
    assert "raised" in out.stdout, out.stderr
