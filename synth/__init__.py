"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This module only draws random numbers and shapes them into the workloads' inputs
(fp32 weights before quantization, BF16 activation rows, MoE routes and router
weights). It contains none of the NVFP4 arithmetic: no encoding, decoding,
scaling or matrix product. Both sides of every parity check consume the arrays it
returns, so an input can never come from the side under test.

Random source: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), used in its counter form: output i of the
stream keyed by ``key`` is ``mix(key + (i + 1) * 0x9E3779B97F4A7C15)``. Normal
variates use the Box-Muller transform in float64.
"""
from .gen import (  # noqa: F401
    splitmix64,
    uniform,
    normal,
    weight_f32,
    act_bf16,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    moe_routes,
    moe_expert_weights,
    WORKLOADS,
)
