"""Seeded synthetic inputs for the one-GPU Mega MoE forward.

This module is shared by the tests, the benchmark and the oracle's callers. It
holds input generation only: random draws, the router's top-k recipe, and the
producer-side casts that turn fp32 draws into the FP8 / FP4 block-scaled input
formats the path consumes. It contains none of the path's own arithmetic
(routing, GEMMs, SwiGLU, requantisation, combine).
"""
from .generate import CONFIGS, MoEConfig, MoEInputs, make_inputs, make_routing, make_weights, make_activations

__all__ = ["CONFIGS", "MoEConfig", "MoEInputs", "make_inputs", "make_routing", "make_weights",
           "make_activations"]
