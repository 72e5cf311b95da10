"""fp64 CPU oracle of streaming chunk-causal attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP library (no kernels, headers,
helpers, tables or pre/post-processing); both sides only consume the same seeded
inputs from the separate `synth` package.

What it computes (StreamRender-H3 project page, "3.1.2 Historical Context and
Temporal Consistency", prefix-cache paragraph, and "3.3 Inference Acceleration
and End-to-End Deployment", static-context KV caching and persistent KV layout):
the current chunk's query tokens attend, with one softmax per row, over the
persistent (reference image + prompt) tokens of the denoising step's bank, the
recent history chunks kept in the rolling window, and the current chunk itself,
bidirectionally inside each causal block of the current chunk.  The method
reaches the plain masked softmax-attention result exactly (the online softmax
only reorders the rounding), so the oracle is that definition written out.

Modules
  native         the plain C++17 fp64 oracle (cpp/attention_oracle.cpp): the definition, its own
                 std::deque cache model and the dense full-sequence route, on std::thread
                 workers; the reference of the GPU parity tests, the smoke check and the
                 benchmark's CPU baseline (loaded on demand: `from oracle import native`)
  attention      masked scaled-dot-product attention, the definition (fp64, numpy)
  cache_model    the streaming cache: persistent banks, rolling window, current chunk
  chunk_attention  one attention call of the current chunk over the cache model
  full_sequence  an independent dense path over the whole stream with an explicit mask
                 (also over one window with the prefix cache's asymmetric mask)
  window_attention  page-literal variant: moving rows over the whole window, prefix rows
                 over their bank
  qk_prep        qk-RMSNorm and rotary embedding of the qkv projection before the cache write
  brute          arbitrary-precision (decimal) brute force for tiny inputs
  mx             MXFP6 (E2M3 + E8M0 block scales) and FP8 E4M3 quantization of the
                 reduced-precision attention's operands
  decoder        the streaming causal decoder's window attention and global-token attention

Every function has at least one pin in tests/test_oracle_pins.py that does not
go through the function itself (closed forms, invariants, brute force, an
independent path).  Parity status: pinned, except where a docstring says
"parity unpinned".
"""
from .attention import masked_attention, widen
from .cache_model import StreamingCache, CacheStateError
from .chunk_attention import chunk_attention, current_block_mask
from .full_sequence import full_sequence_attention, window_full_attention
from .window_attention import window_attention, prefix_attention
from .qk_prep import rms_norm, rope, rope_angles, prep_qkv
from .brute import brute_attention
from .mx import mxfp6_values, fp8_values
from .decoder import decoder_window_attention, decoder_global_attention, window_offsets

__all__ = ["masked_attention", "widen", "StreamingCache", "CacheStateError", "chunk_attention",
           "current_block_mask", "full_sequence_attention", "window_full_attention", "window_attention",
           "prefix_attention", "rms_norm", "rope", "rope_angles", "prep_qkv", "brute_attention",
           "mxfp6_values", "fp8_values",
           "decoder_window_attention", "decoder_global_attention", "window_offsets"]
