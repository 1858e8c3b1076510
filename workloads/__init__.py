"""Seeded synthetic inputs for the routed LoRA delta.

This module only draws numbers: batch structure (per-sequence adapter ids and
lengths), adapter factors in PEFT orientation, activations and the fp32 partial
sums the delta is added to.  It holds none of the delta's arithmetic, so both
the fp64 oracle and the HIP path can take their inputs from it.
"""
from .configs import CONFIGS, config_by_name, LaneSpec, WorkloadSpec
from .gen import (
    Workload, Lane, SliceFactors, Adapter,
    generate, f32_to_bf16_bits, bf16_bits_to_f32, hadamard, draw_fold, draw_base_weight,
)
from .moe import MoeSpec, MoeWorkload, generate_moe, MOE_CONFIGS, moe_config_by_name

__all__ = [
    "CONFIGS", "config_by_name", "LaneSpec", "WorkloadSpec",
    "Workload", "Lane", "SliceFactors", "Adapter",
    "generate", "f32_to_bf16_bits", "bf16_bits_to_f32", "hadamard", "draw_fold",
    "draw_base_weight",
    "MoeSpec", "MoeWorkload", "generate_moe", "MOE_CONFIGS", "moe_config_by_name",
]
