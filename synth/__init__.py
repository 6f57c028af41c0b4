"""Seeded synthetic inputs shared by the CPU oracle and the HIP library.

This package draws data only: random sign words in the library's canonical
packed format, fp16 scale vectors, and bf16/fp32 activations, all from numpy
PCG64 streams keyed by (workload, layer, matrix, path, tensor).  It contains
none of the layer's arithmetic (no packing of +-1 arrays, no reconstruction,
no forward pass, no rank rule).  Ranks are passed in by the caller.
"""
from .gen import (  # noqa: F401
    WORKLOADS,
    MatSpec,
    Workload,
    activations,
    bf16_bits_from_f32,
    int8_signs,
    layer_activations,
    layer_tensors,
    rng_for,
    scales_fp16_bits,
    sign_words,
    signed_scales_fp16_bits,
    wide_range_activations,
)
