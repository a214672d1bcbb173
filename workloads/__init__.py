"""Seeded synthetic inputs for the LatentMoE MXFP4 layer.

This package only draws random inputs (activations, router weights, MXFP4
codes and scales, shared-expert weights, given logits) and packs them into the
byte layouts the layer consumes. It holds none of the layer's arithmetic: no
dequantisation, no routing, no GLU, no combine. Both the CPU oracle and the
GPU tests/bench draw their inputs from here, so both sides see identical bytes.
"""
from .configs import Dims, Workload, WORKLOADS, get_workload
from .gen import (
    gen_x,
    gen_router,
    gen_expert,
    gen_experts,
    gen_shared,
    gen_logits,
    gen_all,
    gen_block,
)

__all__ = [
    "Dims", "Workload", "WORKLOADS", "get_workload",
    "gen_x", "gen_router", "gen_expert", "gen_experts", "gen_shared",
    "gen_logits", "gen_all", "gen_block",
]
