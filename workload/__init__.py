"""Seeded synthetic inputs for the latent-MoE layer.

This package only draws numbers: it holds none of the layer's arithmetic.
Both the CPU oracle (through the tests) and the HIP path (through the tests,
the smoke check and the benchmark) take their inputs from here.
"""
from .gen import (  # noqa: F401
    LayerConfig,
    named_config,
    NAMED_CONFIGS,
    make_x,
    make_dense,
    make_expert,
    make_shared,
    fill_experts,
    expert_record_bytes,
    expert_scale_bytes,
    shared_record_bytes,
    shared_scale_bytes,
    make_router_scores,
    make_selection_bias,
)
