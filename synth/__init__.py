"""Seeded synthetic inputs for the NVFP4 routed-MoE workloads.

This package draws random inputs (BF16 activations and weights, router logits and the routing
they induce) and nothing else: it holds none of the method's arithmetic (no quantization,
plan, projection, activation or combine).  Both the oracle-side tests and the HIP path take
their inputs from here.
"""

from .workloads import (  # noqa: F401
    ACT_NAMES,
    WORKLOADS,
    Workload,
    bf16_bits,
    make_activations,
    make_expert_weight,
    make_routing,
    make_weights,
    to_bits,
)
