"""Seeded synthetic inputs for the one-GPU Mega MoE forward and the standalone FP8 x FP4
GEMMs and FP8 cast.

This module is shared by the tests, the benchmark and the oracle's callers. It
holds input generation only: random draws, the router's top-k recipe, and the
producer-side casts that turn fp32 draws into the FP8 / FP4 block-scaled input
formats the path consumes. It contains none of the path's own arithmetic
(routing, GEMMs, SwiGLU, requantisation, combine). The library's own FP8 cast is checked
against the oracle's cast, never against the generator casts here.
"""
from .generate import (CONFIGS, GEMM_CONFIGS, GemmConfig, GemmInputs, MoEConfig, MoEInputs,
                       make_activations, make_bf16_activations, make_gemm_inputs, make_inputs,
                       make_routing, make_weights)

__all__ = ["CONFIGS", "MoEConfig", "MoEInputs", "make_inputs", "make_routing", "make_weights",
           "make_activations", "GEMM_CONFIGS", "GemmConfig", "GemmInputs", "make_gemm_inputs",
           "make_bf16_activations"]
