"""Seeded synthetic inputs for the gated delta-rule layer and the global attention layer.

This module is shared by the HIP path's tests/benchmark and by the fp64 oracle:
both receive exactly the bytes generated here.  It holds no arithmetic of the
layer itself (no convolution, recurrence or normalisation); it only draws
random numbers with the distributions and shapes of the layer's workloads and
converts them to the storage formats (bf16 bit patterns, fp32) the library
consumes.
"""
from .bf16 import f32_to_bf16_bits, bf16_bits_to_f32
from .configs import (
    LAYER, make_config, decode_step_inputs, varlen_lengths, unit_vectors,
    gate_draws, layer_sequence_inputs, make_layer_config,
)
from .attention import ATTN, attn_prefill_inputs, attn_decode_inputs

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "LAYER", "make_config",
    "decode_step_inputs", "varlen_lengths", "unit_vectors", "gate_draws",
    "layer_sequence_inputs", "make_layer_config",
    "ATTN", "attn_prefill_inputs", "attn_decode_inputs",
]
