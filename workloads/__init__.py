"""Seeded synthetic inputs for the forward-convolution workloads.

This module is shared by the CPU oracle side and the HIP side and holds none
of the convolution's arithmetic: it only describes layer shapes and draws
seeded random tensors, rounded once to the storage dtype.
"""
from .configs import CONFIGS, TABLE1, LayerConfig, get_config, nominal_flops
from .gen import make_inputs, make_config_inputs, make_tensor, round_to_dtype, TORCH_DTYPES

__all__ = [
    "CONFIGS", "TABLE1", "LayerConfig", "get_config", "nominal_flops",
    "make_inputs", "make_config_inputs", "make_tensor", "round_to_dtype", "TORCH_DTYPES",
]
