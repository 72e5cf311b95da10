"""Helpers shared by the tests: build/load the library, move seeded inputs to the device,
run workloads through the C ABI and through the oracle."""
import os

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def lib_module():
    """The binding, building libsr.so first if it is missing."""
    import chunk_causal_attention_amd as sr
    if not os.path.exists(sr.LIB_PATH):
        sr.build()
    sr.load()
    return sr


def cfg_of(sr, w):
    return sr.config_for(w.heads, w.head_dim, w.persistent, w.chunk, w.window, w.causal_block, w.banks,
                         sr.SR_BF16 if w.dtype == "bf16" else sr.SR_F32)


from synth.torch_io import to_dev, to_host  # noqa: E402,F401


def widen_host(arr, dtype):
    if dtype == "bf16":
        return synth.bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def sample_rows(n, tile=256, stride=37, block=None):
    """Rows an oracle can afford at full size: a stride, the ends of every query tile and
    the rows on both sides of every causal-block boundary."""
    rows = set(range(0, n, stride)) | {0, n - 1}
    for t0 in range(0, n, tile):
        rows |= {t0, min(t0 + tile, n) - 1}
    if block and block < n:
        for b in range(block, n, block):
            rows |= {b - 1, b}
    return np.array(sorted(r for r in rows if 0 <= r < n))
