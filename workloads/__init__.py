"""Seeded synthetic inputs for split-KV paged decode attention.

This package only draws random numbers and lays them out (page pools, page
tables, context lengths, bf16 bit patterns).  It holds none of the attention
arithmetic, so both the CPU oracle and the GPU path can take their inputs
from it without sharing any of the method's code.
"""

from .configs import CONFIGS, Workload, get, scaled
from .gen import Inputs, bf16_bits_from_f32, generate

__all__ = ["CONFIGS", "Workload", "get", "scaled", "Inputs", "generate", "bf16_bits_from_f32"]
