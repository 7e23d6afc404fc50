"""Seeded synthetic workloads for the block-canvas denoising step.

This package only describes shapes and draws random inputs. It holds none
of the method's arithmetic: both the CPU oracle (via the tests) and the HIP
path (via the tests and the benchmark) consume what it produces.
"""
from .configs import CONFIGS, Config, get_config
from .inputs import make_inputs, bf16_bits_from_f32, f32_from_bf16_bits

__all__ = ["CONFIGS", "Config", "get_config", "make_inputs",
           "bf16_bits_from_f32", "f32_from_bf16_bits"]
