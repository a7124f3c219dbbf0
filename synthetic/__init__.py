"""Seeded synthetic inputs for the routed-MoE layer (shared by the oracle tests and the GPU path).

This package only *generates* inputs: random weights, activations, router matrices, the
popularity prior and its drift.  It holds none of the layer's arithmetic (no routing, no
decode, no matmul).  The MXFP4 *encoder* used to turn Gaussian weights into expert bytes is
data preparation: both sides only ever decode what it wrote, each with its own decoder.
"""
from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_from_f32,
    quantize_mxfp4,
    expert_canonical,
    router_weights,
    activations,
    zipf_ranks,
    zipf_bias,
    drift_shift,
    experts_canonical,
)
