"""Seeded synthetic inputs for the draft-path selector.

This package is shared by the CPU oracle, the tests and the benchmark.  It only
draws random numbers and lays them out; it holds none of the selector's
arithmetic (no top-k, no gate, no scores, no walk).
"""
from .configs import CONFIGS, Config, config_by_name, variant
from .gen import Inputs, bf16_bits_to_f32, f32_to_bf16_bits, make

__all__ = [
    "CONFIGS",
    "Config",
    "Inputs",
    "bf16_bits_to_f32",
    "config_by_name",
    "f32_to_bf16_bits",
    "make",
    "variant",
]
