"""Seeded synthetic inputs for the routed-MoE expert path.

This module is shared by the CPU oracle's tests and by the HIP path's tests
and benchmark.  It draws random numbers and encodes them into the storage
formats (fp32 router rows, bf16 activations, canonical quantised blocks); it
contains none of the layer's arithmetic (no dequantisation, no routing, no
expert math).
"""

from .workloads import WORKLOADS, Workload, FORMATS, canonical_block_bytes
from .generate import (
    router_weights,
    router_bias,
    expert_canonical,
    layer_canonical,
    shared_canonical,
    token_candidates,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
)

__all__ = [
    "WORKLOADS", "Workload", "FORMATS", "canonical_block_bytes",
    "router_weights", "router_bias", "expert_canonical", "layer_canonical",
    "shared_canonical", "token_candidates", "f32_to_bf16_bits", "bf16_bits_to_f32",
]
