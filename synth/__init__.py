"""Seeded synthetic inputs for the MoE routing-and-balancing layer.

This package only draws random numbers and lays them out; it holds none of
the layer's arithmetic (no gating, no counting, no planning).  Both the CPU
oracle and the GPU path take their inputs from here, so the two sides see
identical bits.
"""
from .workloads import (  # noqa: F401
    CONFIGS,
    MoEConfig,
    LayerInputs,
    config,
    layer_inputs,
    expert_weights,
    shared_weights,
    resident_home,
    scaled,
)
