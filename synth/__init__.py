"""Seeded synthetic inputs for the Beam MoE layer.

This package draws inputs only: activations, router weights, the router bias
column and expert weights (bf16, or e4m3 bytes with per-output-channel fp32
scales). It holds none of the layer's arithmetic (no routing, no expert math,
no combine), so both the CPU oracle and the HIP path can consume it without
sharing any computation.
"""
from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    workload,
    router_inputs,
    redraw_rows,
    guarded_router_inputs,
    expert_matrix,
    ExpertSource,
    bf16_bits,
    bf16_bits_to_f32,
)
