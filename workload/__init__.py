"""Seeded synthetic inputs for the routed-expert MoE layer.

This package is shared by the CPU oracle tests and the HIP path's tests and
benchmark. It holds only the workload shapes, seeded random draws and the
offline INT4 weight preparation (round-to-nearest symmetric quantisation and
nibble packing, which stands in for the GPTQ step of the Specter paper's
draft-model construction). It does none of the layer's arithmetic: routing,
alignment, dequantisation, the expert FFN, the combine and the activation
counter live in `oracle/` (reference) and in the HIP library (product), which
share no code.
"""

from .configs import CONFIGS, MoEConfig, get_config
from .gen import (
    ExpertWeights,
    LayerInputs,
    make_activations,
    make_expert,
    make_layer,
    make_router,
    make_shared,
    pack_int4_codes,
    quantize_rtn_int4,
    zipf_bias,
)

__all__ = [
    "CONFIGS",
    "MoEConfig",
    "get_config",
    "ExpertWeights",
    "LayerInputs",
    "make_activations",
    "make_expert",
    "make_layer",
    "make_router",
    "make_shared",
    "pack_int4_codes",
    "quantize_rtn_int4",
    "zipf_bias",
]
