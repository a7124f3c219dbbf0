"""Seeded synthetic inputs for the routed-MoE layer (shared by the oracle tests and the GPU path).

This package only *generates* inputs: random weights, activations, router matrices, the
popularity prior and its drift.  It holds none of the layer's arithmetic (no routing, no
decode, no matmul).  The MXFP4, FP8 and NVFP4 *encoders* used to turn Gaussian weights into
expert bytes are data preparation: both sides only ever decode what they wrote, each with its
own decoder.
"""
from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_from_f32,
    quantize_mxfp4,
    quantize_fp8_block,
    quantize_nvfp4,
    encode_e4m3,
    expert_canonical,
    router_weights,
    activations,
    zipf_ranks,
    zipf_bias,
    drift_shift,
    experts_canonical,
)
