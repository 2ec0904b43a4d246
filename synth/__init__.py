"""Seeded synthetic inputs for the MXFP4 top-k MoE layer.

This module is shared by the CPU oracle and the GPU path's tests/bench. It holds
no arithmetic of the layer itself: only random draws, bf16 rounding of the drawn
inputs, and the fixed byte layout the inputs are delivered in.
"""
from .generators import (  # noqa: F401
    CONFIGS,
    LayerConfig,
    MoEInputs,
    ExpertWeights,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    AttnInputs,
    make_attn_inputs,
    make_block_x,
    make_inputs,
    make_norm_scale,
    make_x,
    make_expert,
    make_router,
    get_config,
)
