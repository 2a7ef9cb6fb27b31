"""Seeded synthetic inputs for the MoE layer workloads.

This package only draws inputs (token rows, centroids, biases, expert
weights).  It holds none of the layer's arithmetic, so both the CPU oracle
side and the HIP side can consume exactly the same tensors.
"""
from .configs import CONFIGS, LayerConfig, get_config
from .gen import (LayerInputs, make_layer, make_tokens, make_centroids, make_bias,
                  make_expert, bf16_bits, f32_array, host_array, seed_of, HOT_PAIRS)

__all__ = ["CONFIGS", "LayerConfig", "get_config", "LayerInputs", "make_layer",
           "make_tokens", "make_centroids", "make_bias", "make_expert", "bf16_bits",
           "f32_array", "host_array", "seed_of", "HOT_PAIRS"]
