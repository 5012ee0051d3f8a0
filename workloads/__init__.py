"""Seeded synthetic inputs for the XAttention prefill path.

This package only draws random tensors and rounds them to the storage dtype.
It holds none of the method's arithmetic (no scoring, selection or attention),
so both the HIP path's tests/bench and the CPU oracle may use it.
"""
from .configs import CONFIGS, WorkloadConfig, get_config
from .generate import (Workload, generate, bf16_bits_to_f32, f32_to_bf16_bits,
                       as_float64)

__all__ = ["CONFIGS", "WorkloadConfig", "get_config", "Workload", "generate",
           "bf16_bits_to_f32", "f32_to_bf16_bits", "as_float64"]
