"""Seeded synthetic inputs for the MoE expert block.

This module only draws random inputs and describes workload shapes. It holds
none of the expert block's arithmetic (no GEMM, no activation, no permutation,
no quantisation), so both the CPU oracle and the GPU path can take their
inputs from it without sharing any of the method's code.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    Workload,
    make_workload,
    bf16_bits_from_f32,
    bf16_bits_to_f32,
    route_inputs,
)
