"""Routed Mixture-of-Experts layer under expert offloading, for AMD Instinct MI355X (gfx950).

The computation lives in ``libmoe.so`` (hand-written HIP kernels + a C ABI declared in
``include/moe.h``).  ``binding`` exposes the same entry points to Python; ``layer`` holds
device-memory plumbing (slot arrays, workspaces, pinned host banks) built on torch.
"""
from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    MOE_POLICY_LFRU,
    MOE_POLICY_LRU,
    MoeCache,
    MoeError,
    make_shape,
    moe_bucket_routes,
    moe_experts_down,
    moe_experts_forward,
    moe_experts_gateup,
    moe_expert_image_bytes,
    moe_last_error,
    moe_layer_forward,
    moe_pack_expert,
    moe_route,
    moe_slot_refill,
    moe_unpack_expert,
    moe_workspace_size,
)
