"""Seeded synthetic inputs shared by the fp64 oracle and the GPU path.

This package only *draws* numbers: counter-based uniforms, Gaussian deviates,
rounding of the drawn fp32 values to the storage type, and the workload
recipes (shapes, distributions, the AR(1) chunk process, the boosted keys).
It holds none of the attention or cache arithmetic, so both sides of a parity
test consume identical bits without sharing any of the method's code.
"""
from .rng import splitmix64, substream_seed, uniform01, normal, f32_to_bf16_bits, bf16_bits_to_f32
from .workloads import (WORKLOADS, Workload, get_workload, persistent_inputs, SessionStream, WindowStream,
                        single_step_inputs, latent_positions, qkv_inputs, prep_gains,
                        DECODER_WORKLOADS, DecoderWorkload, get_decoder_workload, DecoderStream,
                        window_partition, pack_windows)

__all__ = [
    "splitmix64", "substream_seed", "uniform01", "normal", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "WORKLOADS", "Workload", "get_workload", "persistent_inputs", "SessionStream", "WindowStream",
    "single_step_inputs", "latent_positions", "qkv_inputs", "prep_gains",
    "DECODER_WORKLOADS", "DecoderWorkload", "get_decoder_workload", "DecoderStream",
    "window_partition", "pack_windows",
]
