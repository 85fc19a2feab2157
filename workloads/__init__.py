"""Seeded synthetic workloads for the block-diffusion denoise path.

This package holds the five workload shapes and the seeded generator of their
inputs (weights, prompt KV cache).  It contains none of the method's arithmetic:
both the CPU oracle and the HIP path receive the very tensors it produces.
"""
from .configs import CONFIGS, Config, get_config, tiny_config
from .gen import make_inputs, Inputs

__all__ = ["CONFIGS", "Config", "get_config", "tiny_config", "make_inputs", "Inputs"]
