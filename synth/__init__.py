"""Seeded synthetic inputs shared by the tests, the oracle checks and the benchmark.

This package only draws random numbers and lays tokens out; it holds none of the
mask or attention arithmetic, so the oracle and the HIP path stay independent.
"""
from .configs import CONFIGS, Config, StaSpec, get_config
from .gen import make_inputs, make_signs, token_coords, quantize_fp8_blocks

__all__ = ["CONFIGS", "Config", "StaSpec", "get_config", "make_inputs", "make_signs", "token_coords",
           "quantize_fp8_blocks"]
