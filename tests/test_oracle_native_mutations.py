"""Each plausible mistake planted in a copy of the C++ oracle is caught by a pin (CPU only).

A mutant is the oracle's source with one substitution, compiled into a temporary library; the
real source is untouched.  The pins run against the mutant through the same wrappers
(oracle/native.py) with the mutant library passed in; a mutant "survives" if every pin passes.
Every substitution keeps memory accesses in bounds.
"""
import functools
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import pins
import synth
from oracle import native

# name -> (text in the oracle's source, replacement, replace every occurrence)
MUTANTS = {
    "unscaled_scores": ("s[size_t(r) * nk + j] = scale * dot(", "s[size_t(r) * nk + j] = dot(", False),
    "negated_scores": ("s[size_t(r) * nk + j] = scale * dot(", "s[size_t(r) * nk + j] = -scale * dot(", False),
    "exp2_instead_of_exp": ("std::exp(sr[j] - mx)", "std::exp2(sr[j] - mx)", False),
    "lse_without_max": ("lse[r] = m[r] + std::log(l[r]);", "lse[r] = std::log(l[r]);", False),
    "unnormalised_output": ("o[size_t(r) * Dv + e] /= l[r];", "o[size_t(r) * Dv + e] /= 1.0;", False),
    "mask_ignored": ("visible(r, j)", "(r >= 0 && j >= 0)", True),
    "causal_block_too_wide": ("(rs[r0 + r] / causal_block + 1) * causal_block",
                              "(rs[r0 + r] / causal_block + 2) * causal_block", False),
    "causal_block_too_narrow": ("(rs[r0 + r] / causal_block + 1) * causal_block",
                                "(rs[r0 + r] / causal_block) * causal_block + 1", False),
    "evict_keeps_chunk": ("c.history.pop_front();", "(void)0;", False),
    "commit_drops_chunk": ("c.history.push_back(std::move(c.current));", "(void)0;", False),
    "history_reversed": ("c.history.push_back(std::move(c.current));", "c.history.push_front(std::move(c.current));",
                         False),
    "full_window_not_refused": ("if (int(c.history.size()) == c.window) return 1;", "(void)0;", False),
    "dense_route_window_short": ("if (t < c) return c - t <= window;", "if (t < c) return c - t < window;", False),
    "bf16_widened_wrong": ("const uint32_t u = uint32_t(b) << 16;", "const uint32_t u = (uint32_t(b) << 16) | 0x8000u;",
                           False),
    "update_hits_next_chunk": ("if (h.id == id) {", "if (h.id == id + 1) {", False),
}


def _build(name, tmp):
    old, new, every = MUTANTS[name]
    src = open(native.SOURCE).read()
    assert src.count(old) >= 1, name
    src = src.replace(old, new) if every else src.replace(old, new, 1)
    path = os.path.join(tmp, name + ".cpp")
    with open(path, "w") as f:
        f.write(src)
    lib = os.path.join(tmp, "lib" + name + ".so")
    subprocess.check_call(["g++"] + native.CXXFLAGS + [path, "-o", lib])
    return lib


@pytest.fixture(scope="module")
def mutant_libs(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("oracle_mutants"))
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        paths = dict(zip(MUTANTS, ex.map(lambda n: _build(n, tmp), MUTANTS)))
    return paths


def _cross_check_numpy(L, name="t_frame"):
    """The mutant's stream against the numpy oracle (bf16, boosted keys, frame-causal blocks)."""
    w = synth.get_workload(name)
    stream = synth.SessionStream(w)
    pk, pv = stream.persistent()
    a = oracle.StreamingCache(pk, pv, w.window)
    b = native.StreamingCache(pk, pv, w.window, lib=L)
    for st in stream:
        if st["evict_before"]:
            assert a.evict() == b.evict()
        a.append(st["chunk"], st["k"], st["v"])
        b.append(st["chunk"], st["k"], st["v"])
        oa, la = oracle.chunk_attention(a, 0, st["q"], 0.0884, w.causal_block, w.dtype)
        ob, lb = native.chunk_attention(b, 0, st["q"], 0.0884, w.causal_block, w.dtype)
        assert np.abs(oa - ob).max() <= 1e-12 and np.abs(la - lb).max() <= 1e-12


def _pins(L):
    attn = functools.partial(native.masked_attention, lib=L)
    cache = functools.partial(native.StreamingCache, lib=L)
    full = functools.partial(native.full_sequence_attention, lib=L)
    checks = [functools.partial(p, attn) for p in pins.ALL_ATTENTION_PINS]
    checks += [
        lambda: pins.pin_stream_equals_full_sequence(cache, native.chunk_attention, full),
        lambda: pins.pin_stream_equals_full_sequence(cache, native.chunk_attention, full, window=1, causal_block=2,
                                                     n_chunks=6, seed=12),
        lambda: pins.pin_stream_brute_force(cache, native.chunk_attention),
        lambda: pins.pin_window_rule(cache),
        lambda: pins.pin_update_rule(cache),
        lambda: _cross_check_numpy(L),
    ]
    return checks


def test_real_oracle_passes_every_pin():
    for check in _pins(native.load()):
        check()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(mutant_libs, name):
    L = native.load(mutant_libs[name])
    for check in _pins(L):
        try:
            check()
        except (AssertionError, ValueError, native.CacheStateError):
            return
    pytest.fail("mutant %s survived every pin" % name)
