"""The oracle against what the pages and the mathematics fix (CPU only)."""
import numpy as np
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_ATTENTION_PINS, ids=lambda f: f.__name__)
def test_attention_definition(pin):
    pin(oracle.masked_attention)


def test_stream_equals_full_sequence():
    pins.pin_stream_equals_full_sequence(oracle.StreamingCache, oracle.chunk_attention,
                                         oracle.full_sequence_attention)


@pytest.mark.parametrize("window,cb", [(0, 7), (1, 1), (3, 2)])
def test_stream_equals_full_sequence_shapes(window, cb):
    pins.pin_stream_equals_full_sequence(oracle.StreamingCache, oracle.chunk_attention,
                                         oracle.full_sequence_attention, window=window, causal_block=cb,
                                         n_chunks=7, seed=window * 10 + cb)


def test_stream_brute_force():
    pins.pin_stream_brute_force(oracle.StreamingCache, oracle.chunk_attention)


def test_window_rule():
    pins.pin_window_rule(oracle.StreamingCache)


def test_prefix_rows_see_only_prefix():
    """Prefix rows (building a bank) attend to the prefix alone: equal to masked attention
    over the prefix and independent of anything appended after it."""
    from oracle.full_sequence import prefix_self_attention
    r = np.random.default_rng(5)
    pk, pv, pq = (r.standard_normal((6, 2, 3)).astype(np.float32) for _ in range(3))
    o = prefix_self_attention(pk, pv, pq, 0.5, "f32")
    for h in range(2):
        ref, _ = oracle.masked_attention(pq[:, h].astype(float), pk[:, h].astype(float), pv[:, h].astype(float),
                                         np.ones((6, 6), bool), 0.5)
        assert np.abs(o[:, h] - ref).max() <= 1e-14


def test_masked_future_keys_do_not_matter():
    """Changing keys/values of later causal blocks leaves earlier rows bit-identical."""
    r = np.random.default_rng(9)
    pk = r.standard_normal((1, 4, 2, 8)).astype(np.float32)
    cache = oracle.StreamingCache(pk, pk, 1)
    k, v, q = (r.standard_normal((12, 2, 8)).astype(np.float32) for _ in range(3))
    cache.append(0, k, v)
    o1, l1 = oracle.chunk_attention(cache, 0, q, 0.3, 4, "f32")
    k2, v2 = k.copy(), v.copy()
    k2[8:] = 1e3
    v2[8:] = -7.0
    cache.append(0, k2, v2)
    o2, l2 = oracle.chunk_attention(cache, 0, q, 0.3, 4, "f32")
    assert (o1[:8] == o2[:8]).all() and (l1[:, :8] == l2[:, :8]).all()
    assert not (o1[8:] == o2[8:]).all()


def test_widen_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0001, 0x7F7F, 0xFF80, 0x0000, 0x8000], dtype=np.uint16)
    ref = np.array([1.0, -1.0, 2.0 ** -133, 3.3895313892515355e38, -np.inf, 0.0, -0.0])
    assert (oracle.widen(bits, "bf16") == ref).all()


def test_lse_large_logits_finite():
    """Logits ~1e3 (far past fp32 exp overflow unshifted) stay finite and exact in the max-shift form."""
    q = np.array([[1.0]])
    k = np.array([[1000.0], [999.0]])
    v = np.array([[1.0], [0.0]])
    o, lse = oracle.masked_attention(q, k, v, np.ones((1, 2), bool), 1.0)
    e = np.exp(-1.0)
    assert abs(o[0, 0] - 1.0 / (1.0 + e)) <= 1e-15
    assert abs(lse[0] - (1000.0 + np.log1p(e))) <= 1e-12


def test_window_equals_full_window():
    pins.pin_window_equals_full(oracle.StreamingCache, oracle.window_attention, oracle.prefix_attention,
                                oracle.window_full_attention)


@pytest.mark.parametrize("W", [0, 1, 3])
def test_window_equals_full_window_shapes(W):
    pins.pin_window_equals_full(oracle.StreamingCache, oracle.window_attention, oracle.prefix_attention,
                                oracle.window_full_attention, W=W, n_chunks=6, seed=40 + W)


def test_window_brute_force():
    pins.pin_window_brute_force(oracle.StreamingCache, oracle.window_attention, oracle.prefix_attention)


def test_window_chunking_free():
    pins.pin_window_chunking_free(oracle.StreamingCache, oracle.window_attention)


def test_update_rule():
    pins.pin_update_rule(oracle.StreamingCache)


def test_rms_norm():
    pins.pin_rms_norm(oracle.rms_norm)


def test_rope_closed_form():
    pins.pin_rope_closed_form(oracle.rope)


def test_rope_relative_positions():
    pins.pin_rope_relative(oracle.rope)


def test_rope_sections():
    pins.pin_rope_sections(oracle.rope)


def test_prep_qkv():
    pins.pin_prep_qkv(oracle.prep_qkv, oracle.rms_norm, oracle.rope)


@pytest.mark.parametrize("pin", ["pin_e2m3_values", "pin_e4m3_values", "pin_encode_nearest", "pin_e4m3_encode_torch",
                                 "pin_mx_scale", "pin_mx_quantize"])
def test_mx_quantization(pin):
    """MXFP6 E2M3 / FP8 E4M3 quantization ("The road to the fastest, cheapest H3", reduced
    precision in video attention) against the published formats and brute force."""
    import oracle.mx as mx
    getattr(pins, pin)(mx)


@pytest.mark.parametrize("pin", ["pin_decoder_equals_dense", "pin_decoder_brute", "pin_decoder_window_independence"])
def test_decoder_window_attention(pin):
    """Streaming decoder windows (project page 3.2): per-window routine and global-token routine
    against a dense masked formulation, decimal brute force and window independence."""
    from oracle.decoder import decoder_window_attention, decoder_global_attention
    getattr(pins, pin)(oracle.StreamingCache, decoder_window_attention, decoder_global_attention)


def test_set_bank():
    pins.pin_set_bank(oracle.StreamingCache)
