"""Device-memory plumbing around the C ABI: expert banks, slot arrays, workspaces.

torch is used only to allocate device / pinned-host memory and to name streams; every step
of the layer runs in libmoe's kernels through ``binding``.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B


def pack_bank(shape: B.moe_shape, experts) -> np.ndarray:
    """Pack canonical experts (list of dicts) into a host array [len(experts), image_bytes]."""
    img = B.moe_expert_image_bytes(shape)
    bank = np.empty((len(experts), img), dtype=np.uint8)
    for i, ex in enumerate(experts):
        B.moe_pack_expert(shape, ex, bank[i])
    return bank


def pinned_bank(bank: np.ndarray) -> torch.Tensor:
    """Copy a host bank into page-locked memory (allocated pinned, never registered)."""
    t = torch.empty(bank.shape, dtype=torch.uint8, pin_memory=True)
    t.numpy()[...] = bank
    return t


def device_slots(bank: np.ndarray | torch.Tensor, slot_expert=None, n_slots=None,
                 device="cuda") -> torch.Tensor:
    """Device slot array [n_slots, image_bytes]; slot s holds bank[slot_expert[s]] (or zeros)."""
    img = bank.shape[1]
    if slot_expert is None:
        slot_expert = np.arange(bank.shape[0])
    n_slots = n_slots or len(slot_expert)
    slots = torch.zeros((n_slots, img), dtype=torch.uint8, device=device)
    src = torch.as_tensor(bank) if isinstance(bank, np.ndarray) else bank
    for s, e in enumerate(slot_expert):
        if e >= 0:
            slots[s].copy_(src[int(e)], non_blocking=False)
    return slots


class Buffers:
    """Per-layer device buffers for calls with up to max_M tokens."""

    def __init__(self, shape: B.moe_shape, max_M: int, device="cuda"):
        self.shape = shape
        self.max_M = max_M
        k, H = shape.top_k, shape.hidden
        ws_bytes = B.moe_workspace_size(shape, max_M)
        self.ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=device)
        self.ids = torch.zeros((max(1, max_M), k), dtype=torch.int32, device=device)
        self.w = torch.zeros((max(1, max_M), k), dtype=torch.float32, device=device)
        self.y = torch.zeros((max(1, max_M), H), dtype=torch.float32, device=device)
        self.cold_count = torch.zeros(1, dtype=torch.int32, device=device)
        self.cold_routes = torch.zeros(max(1, max_M * k), dtype=torch.int32, device=device)
