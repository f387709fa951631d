"""Seeded synthetic inputs for the route-layer attention workloads.

This package is shared by the fp64 oracle's tests, the GPU parity tests and the
benchmark. It holds only shapes, seeds and random draws: none of the method's
arithmetic lives here. Every random tensor the method consumes is drawn here and
handed to both sides as identical bits.
"""
from .configs import CONFIGS, Config, get_config
from .gen import (
    bf16_round,
    bf16_to_f64,
    as_f64,
    route_inputs,
    decode_cache,
    decode_step,
    stack_layer_torch,
    sample_query_blocks,
    backward_draws,
)

__all__ = [
    "CONFIGS", "Config", "get_config", "bf16_round", "bf16_to_f64", "as_f64",
    "route_inputs", "decode_cache", "decode_step", "stack_layer_torch",
    "sample_query_blocks", "backward_draws",
]
