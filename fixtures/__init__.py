"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This package holds data generation only (random draws, INT4 packing of the
generated weights, Zipf popularity traces).  It contains none of the layer's
arithmetic: routing, dequantisation, the expert FFN and the combine live in
``oracle/`` (CPU reference) and in the HIP library, which share no code.
"""
from .moe_inputs import (  # noqa: F401
    MoEShape, OLMOE, QWEN_NEXT, seed_of, quantize_int4_g128, pack_int4,
    layer_weights, activations, router_only, zipf_trace,
)
