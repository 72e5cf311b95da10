"""Each plausible mistake planted in a copy of the oracle is caught by at least one pin.

The mutants are written here, on the CPU, as small variants of the oracle's
functions; the real oracle is untouched.  A mutant "survives" if every pin in
its list passes -- that would mean the pins cannot tell it from the real oracle.
"""
import numpy as np
import pytest

import oracle
import pins
from oracle.attention import widen
from oracle.chunk_attention import current_block_mask


def _attn_variant(kind):
    def attn(q, k, v, visible, scale, return_probs=False):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        visible = np.asarray(visible, dtype=bool)
        if kind == "no_scale":
            s = q @ k.T
        elif kind == "sign":
            s = -scale * (q @ k.T)
        elif kind == "dropped_dim":
            s = scale * (q[:, :-1] @ k[:, :-1].T) if q.shape[1] > 1 else scale * 0 * (q @ k.T)
        else:
            s = scale * (q @ k.T)
        if kind != "ignore_mask":
            s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        l = w.sum(axis=1, keepdims=True)
        o = (w @ v) if kind == "no_normalise" else (w @ v) / l
        if kind == "value_transposed" and v.shape[0] == v.shape[1]:
            o = (w @ v.T) / l
        lse = (np.log(l[:, 0]) if kind == "lse_no_max" else m[:, 0] + np.log(l[:, 0]))
        if return_probs:
            return o, lse, w / l if kind != "no_normalise" else w
        return o, lse
    return attn


ATTENTION_MUTANTS = ["no_scale", "sign", "dropped_dim", "ignore_mask", "no_normalise", "lse_no_max"]


def _caught(fn, *args, **kw):
    try:
        fn(*args, **kw)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


@pytest.mark.parametrize("kind", ATTENTION_MUTANTS)
def test_attention_mutant_is_caught(kind):
    attn = _attn_variant(kind)
    assert any(_caught(p, attn) for p in pins.ALL_ATTENTION_PINS), kind


def _chunk_attention_variant(kind):
    def chunk_attn(cache, bank, q, scale, causal_block, dtype):
        if kind == "bank0":
            bank = 0
        k, v, n_fixed = cache.sequence(bank)
        n_cur = k.shape[0] - n_fixed
        rows = np.arange(n_cur)
        H = q.shape[1]
        o = np.zeros((n_cur, H, v.shape[2]))
        lse = np.zeros((H, n_cur))
        for h in range(H):
            if kind == "strict_block":
                cur = (np.arange(n_cur)[None, :] // causal_block) < (rows[:, None] // causal_block)
                cur[np.arange(n_cur), np.arange(n_cur)] = True
            elif kind == "block_off_by_one":
                cur = (np.arange(n_cur)[None, :] // causal_block) <= ((rows[:, None] + 1) // causal_block)
            elif kind == "token_causal":
                cur = np.arange(n_cur)[None, :] <= rows[:, None]
            else:
                cur = current_block_mask(rows, n_cur, causal_block)
            if kind == "history_hidden":
                fixed = np.zeros((n_cur, n_fixed), bool)
                fixed[:, :cache.pk[bank].shape[0]] = True
            else:
                fixed = np.ones((n_cur, n_fixed), bool)
            vis = np.concatenate([fixed, cur], axis=1)
            o[:, h], lse[h] = oracle.masked_attention(widen(q[:, h], dtype), widen(k[:, h], dtype),
                                                      widen(v[:, h], dtype), vis, scale)
        return o, lse
    return chunk_attn


@pytest.mark.parametrize("kind", ["bank0", "strict_block", "block_off_by_one", "token_causal", "history_hidden"])
def test_chunk_attention_mutant_is_caught(kind):
    ca = _chunk_attention_variant(kind)
    assert _caught(pins.pin_stream_equals_full_sequence, oracle.StreamingCache, ca,
                   oracle.full_sequence_attention) or \
        _caught(pins.pin_stream_brute_force, oracle.StreamingCache, ca), kind


class _EvictNewest(oracle.StreamingCache):
    def evict(self):
        if not self.history:
            raise oracle.CacheStateError("empty")
        return self.history.pop()[0]


class _CommitFirstStep(oracle.StreamingCache):
    def append(self, chunk_id, k, v):
        if self.current is not None and chunk_id == self.current[0]:
            return  # keeps the first step's K/V instead of the last
        super().append(chunk_id, k, v)


class _Uncapped(oracle.StreamingCache):
    def append(self, chunk_id, k, v):
        if self.current is not None and chunk_id == self.current[0] + 1 and self.window > 0:
            self.history.append(self.current)
            self.current = (chunk_id, np.array(k), np.array(v))
            return
        super().append(chunk_id, k, v)


class _OrderReversed(oracle.StreamingCache):
    def visible_ids(self):
        return [c for c, _, _ in reversed(self.history)] + ([self.current[0]] if self.current else [])


@pytest.mark.parametrize("cls", [_EvictNewest, _CommitFirstStep, _Uncapped, _OrderReversed],
                         ids=lambda c: c.__name__)
def test_cache_model_mutant_is_caught(cls):
    assert _caught(pins.pin_window_rule, cls) or \
        _caught(pins.pin_stream_equals_full_sequence, cls, oracle.chunk_attention, oracle.full_sequence_attention) \
        or _caught(pins.pin_stream_brute_force, cls, oracle.chunk_attention), cls.__name__


# ---------------------------------------------------------------- page-literal window

def _window_variant(kind):
    """window_attention with a planted mistake in the visible set of the moving rows."""
    def window_attn(cache, bank, q, scale, dtype):
        k, v, _ = cache.sequence(bank)
        P = cache.prefix_len(bank)
        M = k.shape[0] - P
        chunk_of = np.concatenate([np.full(x.shape[0], i) for i, x in
                                   enumerate([h[1] for h in cache.history] + [cache.current[1]])])
        vis = np.ones((M, P + M), bool)
        if kind == "no_current":
            vis[:, P + M - cache.current[1].shape[0]:] = False
            vis[np.arange(M), P + np.arange(M)] = True   # keep every row defined
        elif kind == "chunk_causal":
            vis[:, P:] = chunk_of[None, :] <= chunk_of[:, None]
        elif kind == "no_prefix":
            vis[:, :P] = False
        elif kind == "history_only_own":
            vis[:, P:] = chunk_of[None, :] == chunk_of[:, None]
        H = q.shape[1]
        o = np.zeros((M, H, v.shape[2]))
        lse = np.zeros((H, M))
        for h in range(H):
            o[:, h], lse[h] = oracle.masked_attention(widen(q[:, h], dtype), widen(k[:, h], dtype),
                                                      widen(v[:, h], dtype), vis, scale)
        return o, lse
    return window_attn


@pytest.mark.parametrize("kind", ["no_current", "chunk_causal", "no_prefix", "history_only_own"])
def test_window_mutant_is_caught(kind):
    wa = _window_variant(kind)
    assert _caught(pins.pin_window_equals_full, oracle.StreamingCache, wa, oracle.prefix_attention,
                   oracle.window_full_attention) or \
        _caught(pins.pin_window_brute_force, oracle.StreamingCache, wa, oracle.prefix_attention) or \
        _caught(pins.pin_window_chunking_free, oracle.StreamingCache, wa), kind


def _prefix_sees_window(cache, bank, q, scale, dtype):
    """prefix_attention mutant: the prefix rows also see the moving part."""
    k, v, _ = cache.sequence(bank)
    H = q.shape[1]
    o = np.zeros((q.shape[0], H, v.shape[2]))
    lse = np.zeros((H, q.shape[0]))
    for h in range(H):
        o[:, h], lse[h] = oracle.masked_attention(widen(q[:, h], dtype), widen(k[:, h], dtype), widen(v[:, h], dtype),
                                                  np.ones((q.shape[0], k.shape[0]), bool), scale)
    return o, lse


def test_prefix_mutant_is_caught():
    assert _caught(pins.pin_window_equals_full, oracle.StreamingCache, oracle.window_attention, _prefix_sees_window,
                   oracle.window_full_attention)


class _UpdateCurrentOnly(oracle.StreamingCache):
    def update(self, chunk_id, k, v):
        if self.current is not None and chunk_id == self.current[0]:
            self.current = (chunk_id, np.array(k), np.array(v))
        elif chunk_id not in [c for c, _, _ in self.history]:
            raise oracle.CacheStateError("not in the window")


class _UpdateOldest(oracle.StreamingCache):
    def update(self, chunk_id, k, v):
        if self.history and chunk_id != self.current[0]:
            cid = self.history[0][0]
            self.history[0] = (cid, np.array(k), np.array(v))
            return
        super().update(chunk_id, k, v)


class _UpdateAnyId(oracle.StreamingCache):
    def update(self, chunk_id, k, v):
        try:
            super().update(chunk_id, k, v)
        except oracle.CacheStateError:
            self.current = (self.current[0], np.array(k), np.array(v))


@pytest.mark.parametrize("cls", [_UpdateCurrentOnly, _UpdateOldest, _UpdateAnyId], ids=lambda c: c.__name__)
def test_update_mutant_is_caught(cls):
    assert _caught(pins.pin_update_rule, cls) or \
        _caught(pins.pin_window_equals_full, cls, oracle.window_attention, oracle.prefix_attention,
                oracle.window_full_attention), cls.__name__


# ---------------------------------------------------------------- qk-RMSNorm + rotary embedding

def _rms_variant(kind):
    def rms_norm(x, gamma, eps):
        x = np.asarray(x, dtype=np.float64)
        ms = np.sum(x * x, axis=-1, keepdims=True) if kind == "sum" else np.mean(x * x, axis=-1, keepdims=True)
        if kind == "eps_outside":
            return x / (np.sqrt(ms) + eps) * np.asarray(gamma, dtype=np.float64)
        if kind == "no_gamma":
            return x / np.sqrt(ms + eps)
        return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)
    return rms_norm


@pytest.mark.parametrize("kind", ["sum", "eps_outside", "no_gamma"])
def test_rms_norm_mutant_is_caught(kind):
    assert _caught(pins.pin_rms_norm, _rms_variant(kind)), kind


def _rope_variant(kind):
    from oracle.qk_prep import rope_angles

    def rope(x, pos, sections, base):
        x = np.asarray(x, dtype=np.float64)
        if kind == "exponent":
            pos_ = np.asarray(pos, dtype=np.float64)
            cols = []
            for a, n_a in enumerate(sections):
                k = np.arange(n_a, dtype=np.float64)
                cols.append(pos_[:, a:a + 1] * np.power(float(base), -2 * k / n_a)[None, :])
            ang = np.concatenate(cols, axis=1)[:, None, :]
        elif kind == "axes_swapped":
            ang = rope_angles(np.asarray(pos)[:, [1, 0, 2]], sections, base)[:, None, :]
        else:
            ang = rope_angles(pos, sections, base)[:, None, :]
        c, s = np.cos(ang), np.sin(ang)
        if kind == "sign":
            s = -s
        out = np.empty_like(x)
        if kind == "rotate_half":
            h = x.shape[-1] // 2
            a, b = x[..., :h], x[..., h:]
            out[..., :h] = a * c - b * s
            out[..., h:] = a * s + b * c
            return out
        a, b = x[..., 0::2], x[..., 1::2]
        out[..., 0::2] = a * c - b * s
        out[..., 1::2] = a * s + b * c
        return out
    return rope


@pytest.mark.parametrize("kind", ["exponent", "axes_swapped", "sign", "rotate_half"])
def test_rope_mutant_is_caught(kind):
    rp = _rope_variant(kind)
    assert _caught(pins.pin_rope_closed_form, rp) or _caught(pins.pin_rope_relative, rp) or \
        _caught(pins.pin_rope_sections, rp), kind


def _prep_rotate_then_norm(qkv, pos, gamma_q, gamma_k, eps, sections, base, dtype):
    q, k, v = (widen(qkv[:, i], dtype) for i in range(3))
    return (oracle.rms_norm(oracle.rope(q, pos, sections, base), gamma_q, eps),
            oracle.rms_norm(oracle.rope(k, pos, sections, base), gamma_k, eps), v)


def _prep_shared_gain(qkv, pos, gamma_q, gamma_k, eps, sections, base, dtype):
    return oracle.prep_qkv(qkv, pos, gamma_q, gamma_q, eps, sections, base, dtype)


@pytest.mark.parametrize("fn", [_prep_rotate_then_norm, _prep_shared_gain], ids=lambda f: f.__name__)
def test_prep_mutant_is_caught(fn):
    assert _caught(pins.pin_prep_qkv, fn, oracle.rms_norm, oracle.rope)


# ---------------------------------------------------------------- MXFP6 / FP8 quantization
# Mutants replace one function of oracle.mx for the duration of a test (monkeypatch), so the
# module's other functions (decode, mx_quantize, fp8_values) pick the mistake up too.

import oracle.mx as mx  # noqa: E402

MX_PINS = [pins.pin_e2m3_values, pins.pin_e4m3_values, pins.pin_encode_nearest, pins.pin_e4m3_encode_torch,
           pins.pin_mx_scale, pins.pin_mx_quantize]


def _element_value_variant(kind):
    def element_value(code, fmt):
        eb, mb, bias, _ = fmt
        if kind == "e2m3_bias0" and fmt == mx.E2M3:
            bias = 0
        width = 1 + eb + mb
        sign = -1.0 if (int(code) >> (width - 1)) & 1 else 1.0
        e = (int(code) >> mb) & ((1 << eb) - 1)
        m = int(code) & ((1 << mb) - 1)
        if fmt == mx.E4M3 and e == 15 and m == 7 and kind != "no_nan":
            return float("nan")
        if e == 0:
            return sign * (m / 2.0 ** mb) * 2.0 ** ((-bias) if kind == "subnormal_exp" else (1 - bias))
        return sign * (1.0 + m / 2.0 ** mb) * 2.0 ** (e - bias)
    return element_value


def _encode_variant(kind):
    def encode(x, fmt):
        eb, mb, bias, vmax = fmt
        x = np.asarray(x, dtype=np.float64)
        a = np.abs(x)
        emin = (-bias) if kind == "subnormal_quantum" else 1 - bias
        _, fe = np.frexp(a)
        ex = np.maximum(np.where(a > 0, fe - 1, emin), emin).astype(np.float64)
        quantum = np.exp2(ex - mb)
        if kind == "truncate":
            r = np.floor(a / quantum) * quantum
        elif kind == "ties_away":
            r = np.floor(a / quantum + 0.5) * quantum
        else:
            r = np.rint(a / quantum) * quantum
        if kind != "no_saturate":
            r = np.minimum(r, vmax)
        emin = 1 - bias
        sub = r < 2.0 ** emin
        m_sub = np.rint(r / 2.0 ** (emin - mb))
        _, re = np.frexp(np.where(sub, 1.0, r))
        m_norm = np.rint((np.where(sub, 1.0, r) / np.exp2(re - 1) - 1.0) * 2 ** mb)
        e_field = np.where(sub, 0, re - 1 + bias).astype(np.int64)
        m_field = np.where(sub, m_sub, m_norm).astype(np.int64)
        sign = np.zeros(x.shape, np.int64) if kind == "drop_sign" else np.signbit(x).astype(np.int64)
        return (((sign << (eb + mb)) | (e_field << mb) | m_field) & 0xFF).astype(np.uint8)
    return encode


def _scale_variant(kind):
    def mx_scale_exponents(x):
        x = np.asarray(x, dtype=np.float64)
        blk = 16 if kind == "block16" else 32
        blocks = x.reshape(x.shape[:-1] + (x.shape[-1] // blk, blk))
        amax = np.abs(blocks).max(axis=-1)
        if kind == "row_amax":
            amax = np.repeat(amax.max(axis=-1, keepdims=True), amax.shape[-1], axis=-1)
        _, fe = np.frexp(amax)
        fl = fe - 1
        if kind == "ceil":
            fl = np.where(amax == np.exp2(fl), fl, fl + 1)
        X = np.where(amax > 0, fl - (3 if kind == "emax3" else 2), -127)
        return (X if kind == "no_clamp" else np.clip(X, -127, 127)).astype(np.int64)
    return mx_scale_exponents


MX_MUTANTS = ([("element_value", k, _element_value_variant(k)) for k in ("e2m3_bias0", "subnormal_exp", "no_nan")] +
              [("encode", k, _encode_variant(k)) for k in ("truncate", "ties_away", "no_saturate", "drop_sign",
                                                           "subnormal_quantum")] +
              [("mx_scale_exponents", k, _scale_variant(k)) for k in ("emax3", "ceil", "block16", "row_amax",
                                                                      "no_clamp")])


@pytest.mark.parametrize("name,kind,fn", MX_MUTANTS, ids=[f"{n}-{k}" for n, k, _ in MX_MUTANTS])
def test_mx_mutant_is_caught(monkeypatch, name, kind, fn):
    monkeypatch.setattr(mx, name, fn)
    assert any(_caught(p, mx) for p in MX_PINS), (name, kind)


# ---------------------------------------------------------------- streaming decoder window attention

from oracle.decoder import decoder_window_attention, decoder_global_attention, window_rows  # noqa: E402


def _decoder_window_variant(kind):
    def win_attn(cache, window_tokens, frames, q, scale, dtype):
        T = q.shape[0]
        gk, gv = cache.pk[0], cache.pv[0]
        hist = [(k, v) for _, k, v in cache.history]
        chunks = ([] if kind == "no_history" else hist) + [(cache.current[1], cache.current[2])]
        H = q.shape[1]
        o = np.zeros((T, H, q.shape[2]))
        lse = np.zeros((H, T))
        n_win = len(window_tokens)
        for w in range(n_win):
            rows = window_rows(window_tokens, frames, w)
            if kind == "frame_major":   # window rows taken from a frame-by-frame layout
                per = np.asarray(window_tokens)
                start = int(per[:w].sum())
                rows = np.concatenate([f * int(per.sum()) + start + np.arange(per[w]) for f in range(frames)])
            krows = np.arange(T) if kind == "all_windows" else rows
            parts_k = ([] if kind == "no_global" else [gk]) + [k[krows] for k, _ in chunks]
            parts_v = ([] if kind == "no_global" else [gv]) + [v[krows] for _, v in chunks]
            keys, vals = np.concatenate(parts_k), np.concatenate(parts_v)
            for h in range(H):
                o[rows, h], lse[h, rows] = oracle.masked_attention(widen(q[rows, h], dtype), widen(keys[:, h], dtype),
                                                                   widen(vals[:, h], dtype),
                                                                   np.ones((len(rows), keys.shape[0]), bool), scale)
        return o, lse
    return win_attn


def _decoder_global_sees_history(cache, gq, scale, dtype):
    keys = np.concatenate([cache.pk[0]] + [k for _, k, _ in cache.history] + [cache.current[1]])
    vals = np.concatenate([cache.pv[0]] + [v for _, _, v in cache.history] + [cache.current[2]])
    H = gq.shape[1]
    o = np.zeros((gq.shape[0], H, gq.shape[2]))
    lse = np.zeros((H, gq.shape[0]))
    for h in range(H):
        o[:, h], lse[h] = oracle.masked_attention(widen(gq[:, h], dtype), widen(keys[:, h], dtype),
                                                  widen(vals[:, h], dtype), np.ones((gq.shape[0], keys.shape[0]), bool),
                                                  scale)
    return o, lse


DECODER_PINS = [pins.pin_decoder_equals_dense, pins.pin_decoder_brute, pins.pin_decoder_window_independence]


@pytest.mark.parametrize("kind", ["all_windows", "no_history", "no_global", "frame_major"])
def test_decoder_window_mutant_is_caught(kind):
    wa = _decoder_window_variant(kind)
    assert any(_caught(p, oracle.StreamingCache, wa, decoder_global_attention) for p in DECODER_PINS), kind


def test_decoder_global_mutant_is_caught():
    assert any(_caught(p, oracle.StreamingCache, decoder_window_attention, _decoder_global_sees_history)
               for p in DECODER_PINS)


class _SetBankZero(oracle.StreamingCache):
    def set_bank(self, bank, k, v):
        super().set_bank(0, k, v)


@pytest.mark.parametrize("cls", [_SetBankZero], ids=lambda c: c.__name__)
def test_set_bank_mutant_is_caught(cls):
    assert _caught(pins.pin_set_bank, cls)
