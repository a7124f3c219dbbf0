"""ctypes binding of libmoe (include/moe.h): the same entry points, argument marshalling only.

Every computation happens in the HIP library; this module converts torch tensors (device
pointers), numpy arrays (host pointers), streams and events into C arguments and turns a
non-OK status into an exception.  If libmoe.so is missing the import fails loudly: there is no
other implementation to fall back to.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_HIP = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_STATE = -5
MOE_POLICY_LRU = 0
MOE_POLICY_LFRU = 1


class MoeError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func} failed with status {status}: {msg}")
        self.status = status


class moe_shape(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("inter", C.c_int32), ("n_experts", C.c_int32),
                ("top_k", C.c_int32), ("n_slots", C.c_int32), ("format", C.c_int32)]


MOE_FORMAT_MXFP4, MOE_FORMAT_BF16, MOE_FORMAT_FP8_BLOCK, MOE_FORMAT_NVFP4 = 0, 1, 2, 3
FORMAT_IDS = {"mxfp4": MOE_FORMAT_MXFP4, "bf16": MOE_FORMAT_BF16,
              "fp8_block": MOE_FORMAT_FP8_BLOCK, "nvfp4": MOE_FORMAT_NVFP4}


class moe_cache_config(C.Structure):
    _fields_ = [("policy", C.c_int32), ("max_refills_per_step", C.c_int32),
                ("lag_steps", C.c_int32), ("max_pending", C.c_int32),
                ("decay_period", C.c_int32)]


class moe_refill(C.Structure):
    _fields_ = [("expert", C.c_int32), ("slot", C.c_int32), ("evicted", C.c_int32),
                ("reserved", C.c_int32), ("visible_step", C.c_int64)]


class moe_hybrid_staging(C.Structure):
    _fields_ = [("max_M", C.c_int32), ("x", C.c_void_p), ("ids", C.c_void_p), ("w", C.c_void_p),
                ("y_cold", C.c_void_p), ("y_cold_dev", C.c_void_p), ("routed", C.c_void_p),
                ("added", C.c_void_p), ("pending", C.c_int32)]


class moe_prefill_staging(C.Structure):
    _fields_ = [("max_M", C.c_int32), ("n_slots", C.c_int32), ("slots", C.c_void_p),
                ("counts_dev", C.c_void_p), ("counts_host", C.c_void_p), ("maps_dev", C.c_void_p),
                ("maps_host", C.c_void_p), ("y_pass", C.c_void_p), ("copy_stream", C.c_void_p),
                ("ev_counts", C.c_void_p), ("ev_copied", C.c_void_p * 2), ("ev_done", C.c_void_p * 2),
                ("pending", C.c_int32 * 2)]


class moe_cache_stats(C.Structure):
    _fields_ = [("steps", C.c_int64), ("routes", C.c_int64), ("hits", C.c_int64),
                ("refills", C.c_int64), ("evictions", C.c_int64)]


_P = C.c_void_p
_I32 = C.c_int32
_SZ = C.c_size_t
_SIGS = {
    "moe_expert_image_bytes": [C.POINTER(moe_shape), C.POINTER(_SZ)],
    "moe_pack_expert": [C.POINTER(moe_shape)] + [_P] * 7,
    "moe_unpack_expert": [C.POINTER(moe_shape)] + [_P] * 7,
    "moe_workspace_size": [C.POINTER(moe_shape), _I32, C.POINTER(_SZ)],
    "moe_route": [C.POINTER(moe_shape), _P, _I32, _P, _P, _P, _P, _P, _SZ, _P],
    "moe_bucket_routes": [C.POINTER(moe_shape), _P, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "moe_experts_forward": [C.POINTER(moe_shape), _P, _I32, _P, _P, _P, _P, _P, _P, _P, _P,
                            _SZ, _P],
    "moe_layer_forward": [C.POINTER(moe_shape), _P, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                          _P, _SZ, _P],
    "moe_layer_forward_marked": [C.POINTER(moe_shape), _P, _I32, _P, _P, _P, _P, _P, _P, _P, _P,
                                 _P, _P, _SZ, _P, _P],
    "moe_layer_forward_residual": [C.POINTER(moe_shape), _P, _I32, _P, _P, _P, _P, _P, _P, _P, _P,
                                   _P, _P, _P, _SZ, _P],
    "moe_layer_launches": [C.POINTER(moe_shape), _I32, C.POINTER(_I32)],
    "moe_experts_gateup": [C.POINTER(moe_shape), _P, _I32, _P, _P, _P, _P, _P, _SZ, _P],
    "moe_experts_down": [C.POINTER(moe_shape), _I32, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "moe_slot_refill": [C.POINTER(moe_shape), _P, _P, _P, _P, _I32, _P, _P, _P],
    "moe_residual_bf16": [_P, _P, _P, _SZ, _P],
    "moe_workspace_errors": [_P, _SZ, _P, _P],
    "moe_device_cache_size": [C.POINTER(moe_shape), C.POINTER(_SZ)],
    "moe_device_cache_init": [C.POINTER(moe_shape), C.POINTER(moe_cache_config), _P, C.c_int64, _P,
                              _SZ, _P],
    "moe_device_cache_step": [C.POINTER(moe_shape), _P, _SZ, _P, _I32, _P, _P, _P, _P],
    "moe_device_cache_copy": [C.POINTER(moe_shape), _P, _P, _P, _P, _P],
    "moe_device_cache_stats": [C.POINTER(moe_shape), _P, _SZ, _P, _P],
    "moe_layer_forward_staged": [C.POINTER(moe_shape), _P, _I32, _P, _P, _P, _P, _P, _P,
                                 C.POINTER(moe_prefill_staging), _P, _SZ, _P, C.POINTER(_I32),
                                 C.POINTER(_I32)],
    "moe_hbm_read_probe": [_P, _SZ, _P, _P],
    "moe_cold_forward_host": [C.POINTER(moe_shape), _P, _P, _I32, _P, _P, _P, _P, _I32],
    "moe_layer_forward_hybrid": [C.POINTER(moe_shape), _P, _I32, _P, _P, _P, _P, _P, _P, _P, _P,
                                 _P, C.POINTER(moe_hybrid_staging), _I32, _P, _SZ, _P],
    "moe_layer_forward_noalloc": [C.POINTER(moe_shape), _P, _I32, _P, _P, _P, _P, _P, _P, _P, _P,
                                  _P, _P, _P],
    "moe_cache_create": [C.POINTER(moe_shape), C.POINTER(moe_cache_config), _P,
                         C.POINTER(_P)],
    "moe_cache_policy_step": [_P, C.c_int64, _P, _I32, _P, C.POINTER(_I32), _P,
                              C.POINTER(moe_cache_stats)],
    "moe_cache_state_bytes": [_P, C.POINTER(_SZ)],
    "moe_cache_save": [_P, _P, _SZ],
    "moe_cache_restore": [_P, _P, _SZ],
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libmoe.so (once).  Raises if the library has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m expert_offloaded_routed_amd._build`")
    # torch carries its own HIP runtime; load it first so that libmoe binds to the same one
    # (two runtimes in one process do not share devices, streams or allocations).
    import torch  # noqa: F401
    lib = C.CDLL(path)
    for name, argtypes in _SIGS.items():
        f = getattr(lib, name)
        f.argtypes = argtypes
        f.restype = C.c_int
    lib.moe_cache_destroy.argtypes = [_P]
    lib.moe_cache_destroy.restype = None
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = C.c_char_p
    _lib = lib
    return lib


def moe_last_error() -> str:
    return load().moe_last_error().decode()


def _check(status: int, func: str):
    if status != MOE_OK:
        raise MoeError(status, func, moe_last_error())


# ---------------------------------------------------------------------------------------------
# argument conversion
# ---------------------------------------------------------------------------------------------
def _ptr(a):
    """torch tensor -> data_ptr, numpy array -> host address, int -> itself, None -> NULL."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    if isinstance(a, np.ndarray):
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("numpy argument must be C-contiguous")
        return a.ctypes.data
    dp = getattr(a, "data_ptr", None)
    if dp is not None:
        if not a.is_contiguous():
            raise ValueError("tensor argument must be contiguous")
        return dp()
    raise TypeError(f"cannot pass {type(a)} as a pointer")


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _nbytes(a):
    if isinstance(a, np.ndarray):
        return a.nbytes
    return a.numel() * a.element_size()


def make_shape(hidden, inter, n_experts, top_k, n_slots, fmt="mxfp4") -> moe_shape:
    """fmt: a moe_format value or its name ("mxfp4", "bf16", "fp8_block", "nvfp4")."""
    return moe_shape(hidden, inter, n_experts, top_k, n_slots,
                     FORMAT_IDS[fmt] if isinstance(fmt, str) else int(fmt))


_NAMES = ("gate_codes", "gate_scales", "up_codes", "up_scales", "down_codes", "down_scales")


def _format_arrays(shape: moe_shape, expert: dict) -> list:
    """The six byte arrays moe_pack_expert takes for the shape's format (None = NULL).

    Expert dicts of the other formats: *_codes = elements (bf16 as uint16, E4M3 / E2M1 codes as
    uint8); *_scales = fp32 block scales (FP8 block) or E4M3 bytes [N, K/16] (NVFP4, whose
    fp32 matrix scale is *_global)."""
    f = shape.format
    out = []
    for name in _NAMES:
        mat, kind = name.split("_")
        if kind == "codes":
            a = np.ascontiguousarray(expert[name])
            out.append(a.reshape(-1).view(np.uint8))
        elif f == MOE_FORMAT_MXFP4:
            out.append(np.ascontiguousarray(expert[name], dtype=np.uint8).reshape(-1))
        elif f == MOE_FORMAT_BF16:
            out.append(None)
        elif f == MOE_FORMAT_FP8_BLOCK:
            out.append(np.ascontiguousarray(expert[name], dtype=np.float32).reshape(-1).view(np.uint8))
        else:
            g = np.asarray([expert[mat + "_global"]], dtype=np.float32).view(np.uint8)
            out.append(np.concatenate([g, np.ascontiguousarray(expert[name], dtype=np.uint8).reshape(-1)]))
    return out


# ---------------------------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------------------------
def moe_expert_image_bytes(shape: moe_shape) -> int:
    out = _SZ(0)
    _check(load().moe_expert_image_bytes(C.byref(shape), C.byref(out)), "moe_expert_image_bytes")
    return out.value


def moe_pack_expert(shape: moe_shape, expert: dict, image: np.ndarray | None = None) -> np.ndarray:
    """Canonical MXFP4 dict (gate/up/down codes+scales, numpy uint8) -> image (numpy uint8)."""
    n = moe_expert_image_bytes(shape)
    if image is None:
        image = np.empty(n, dtype=np.uint8)
    if image.nbytes < n:
        raise ValueError("image buffer too small")
    args = _format_arrays(shape, expert)
    _check(load().moe_pack_expert(C.byref(shape), *[None if a is None else _ptr(a) for a in args],
                                  _ptr(image)), "moe_pack_expert")
    return image


def moe_unpack_expert(shape: moe_shape, image: np.ndarray) -> dict:
    H, I = shape.hidden, shape.inter
    if shape.format != MOE_FORMAT_MXFP4:
        return _unpack_format(shape, image)
    out = {"gate_codes": np.empty((I, H // 2), np.uint8), "gate_scales": np.empty((I, H // 32), np.uint8),
           "up_codes": np.empty((I, H // 2), np.uint8), "up_scales": np.empty((I, H // 32), np.uint8),
           "down_codes": np.empty((H, I // 2), np.uint8), "down_scales": np.empty((H, I // 32), np.uint8)}
    _check(load().moe_unpack_expert(C.byref(shape), _ptr(np.ascontiguousarray(image)),
                                    *[_ptr(out[k]) for k in ("gate_codes", "gate_scales", "up_codes",
                                                             "up_scales", "down_codes", "down_scales")]),
           "moe_unpack_expert")
    return out


def _unpack_format(shape: moe_shape, image: np.ndarray) -> dict:
    H, I, f = shape.hidden, shape.inter, shape.format
    dims = {"gate": (I, H), "up": (I, H), "down": (H, I)}
    bufs, out = [], {}
    for name in _NAMES:
        mat, kind = name.split("_")
        n, k = dims[mat]
        if kind == "codes":
            a = np.empty((n, k), np.uint16) if f == MOE_FORMAT_BF16 else \
                np.empty((n, k if f == MOE_FORMAT_FP8_BLOCK else k // 2), np.uint8)
            out[name] = a
            bufs.append(a)
        elif f == MOE_FORMAT_BF16:
            bufs.append(None)
        elif f == MOE_FORMAT_FP8_BLOCK:
            a = np.empty(((n + 127) // 128, (k + 127) // 128), np.float32)
            out[name] = a
            bufs.append(a)
        else:
            a = np.empty(4 + n * (k // 16), np.uint8)
            bufs.append(a)
    _check(load().moe_unpack_expert(C.byref(shape), _ptr(np.ascontiguousarray(image)),
                                    *[None if b is None else _ptr(b) for b in bufs]),
           "moe_unpack_expert")
    if f == MOE_FORMAT_NVFP4:
        for i, name in enumerate(_NAMES):
            if name.endswith("_scales"):
                mat = name.split("_")[0]
                n, k = dims[mat]
                out[mat + "_global"] = float(bufs[i][:4].view(np.float32)[0])
                out[name] = bufs[i][4:].reshape(n, k // 16).copy()
    return out


def moe_workspace_size(shape: moe_shape, max_M: int) -> int:
    out = _SZ(0)
    _check(load().moe_workspace_size(C.byref(shape), int(max_M), C.byref(out)), "moe_workspace_size")
    return out.value


def moe_route(shape, x, M, w_router, router_bias, topk_ids, topk_w, ws, stream=None):
    _check(load().moe_route(C.byref(shape), _ptr(x), int(M), _ptr(w_router), _ptr(router_bias),
                            _ptr(topk_ids), _ptr(topk_w), _ptr(ws), _nbytes(ws), _stream(stream)),
           "moe_route")


def moe_bucket_routes(shape, topk_ids, M, expert_to_slot, counts, offsets, perm, cold_count,
                      cold_routes, ws, stream=None):
    _check(load().moe_bucket_routes(C.byref(shape), _ptr(topk_ids), int(M), _ptr(expert_to_slot),
                                    _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(cold_count),
                                    _ptr(cold_routes), _ptr(ws), _nbytes(ws), _stream(stream)),
           "moe_bucket_routes")


def moe_experts_forward(shape, x, M, topk_ids, topk_w, expert_to_slot, slots, y, cold_count,
                        cold_routes, ws, stream=None):
    _check(load().moe_experts_forward(C.byref(shape), _ptr(x), int(M), _ptr(topk_ids),
                                      _ptr(topk_w), _ptr(expert_to_slot), _ptr(slots), _ptr(y),
                                      _ptr(cold_count), _ptr(cold_routes), _ptr(ws), _nbytes(ws),
                                      _stream(stream)),
           "moe_experts_forward")


def moe_layer_forward(shape, x, M, w_router, router_bias, expert_to_slot, slots, topk_ids, topk_w,
                      y, cold_count, cold_routes, ws, stream=None):
    _check(load().moe_layer_forward(C.byref(shape), _ptr(x), int(M), _ptr(w_router),
                                    _ptr(router_bias), _ptr(expert_to_slot), _ptr(slots),
                                    _ptr(topk_ids), _ptr(topk_w), _ptr(y), _ptr(cold_count),
                                    _ptr(cold_routes), _ptr(ws), _nbytes(ws), _stream(stream)),
           "moe_layer_forward")


def moe_layer_forward_residual(shape, x, M, w_router, router_bias, expert_to_slot, slots, topk_ids,
                               topk_w, y, cold_count, cold_routes, x_next, ws, stream=None):
    """moe_layer_forward that also writes x_next = bf16(x + y) (x_next may be x)."""
    _check(load().moe_layer_forward_residual(C.byref(shape), _ptr(x), int(M), _ptr(w_router),
                                             _ptr(router_bias), _ptr(expert_to_slot), _ptr(slots),
                                             _ptr(topk_ids), _ptr(topk_w), _ptr(y), _ptr(cold_count),
                                             _ptr(cold_routes), _ptr(x_next), _ptr(ws), _nbytes(ws),
                                             _stream(stream)),
           "moe_layer_forward_residual")


def moe_layer_forward_noalloc(shape, x, M, w_router, router_bias, expert_to_slot, slots, topk_ids,
                              topk_w, y, cold_count, cold_routes, errors=None, stream=None):
    """moe_layer_forward on the library's static scratch (no workspace argument, no allocation)."""
    _check(load().moe_layer_forward_noalloc(C.byref(shape), _ptr(x), int(M), _ptr(w_router),
                                            _ptr(router_bias), _ptr(expert_to_slot), _ptr(slots),
                                            _ptr(topk_ids), _ptr(topk_w), _ptr(y), _ptr(cold_count),
                                            _ptr(cold_routes), _ptr(errors), _stream(stream)),
           "moe_layer_forward_noalloc")


def moe_layer_forward_marked(shape, x, M, w_router, router_bias, expert_to_slot, slots, topk_ids,
                             topk_w, y, cold_count, cold_routes, ws, marks, stream=None):
    """moe_layer_forward with four HIP events recorded at its stage boundaries."""
    ev = (C.c_void_p * 4)(*[C.c_void_p(int(m)) for m in marks])
    _check(load().moe_layer_forward_marked(C.byref(shape), _ptr(x), int(M), _ptr(w_router),
                                           _ptr(router_bias), _ptr(expert_to_slot), _ptr(slots),
                                           _ptr(topk_ids), _ptr(topk_w), _ptr(y), _ptr(cold_count),
                                           _ptr(cold_routes), _ptr(ws), _nbytes(ws), _stream(stream),
                                           C.cast(ev, C.c_void_p)),
           "moe_layer_forward_marked")


def moe_layer_launches(shape, M):
    """Kernel launches of one moe_layer_forward call for M tokens (2 = gate/up and down fused)."""
    n = _I32(0)
    _check(load().moe_layer_launches(C.byref(shape), int(M), C.byref(n)), "moe_layer_launches")
    return int(n.value)


def moe_experts_gateup(shape, x, M, topk_ids, topk_w, expert_to_slot, slots, ws, stream=None):
    _check(load().moe_experts_gateup(C.byref(shape), _ptr(x), int(M), _ptr(topk_ids), _ptr(topk_w),
                                     _ptr(expert_to_slot), _ptr(slots), _ptr(ws), _nbytes(ws),
                                     _stream(stream)), "moe_experts_gateup")


def moe_experts_down(shape, M, topk_ids, topk_w, expert_to_slot, slots, y, ws, stream=None):
    _check(load().moe_experts_down(C.byref(shape), int(M), _ptr(topk_ids), _ptr(topk_w),
                                   _ptr(expert_to_slot), _ptr(slots), _ptr(y), _ptr(ws),
                                   _nbytes(ws), _stream(stream)), "moe_experts_down")


MOE_DEVERR_BAD_ID = 1
MOE_DEVERR_BAD_SLOT = 2
MOE_DEVERR_HANDOFF = 4


def moe_workspace_errors(ws, flags, stream=None):
    """Enqueue a copy of the workspace's device error word into ``flags`` (one int32, device or
    pinned host memory)."""
    _check(load().moe_workspace_errors(_ptr(ws), _nbytes(ws), _ptr(flags), _stream(stream)),
           "moe_workspace_errors")


def moe_cold_forward_host(shape, host_bank, x, M, topk_ids, topk_w, expert_to_slot, y_cold,
                          n_threads=0):
    """The cold routes of a call on the host cores (every array a host numpy array)."""
    _check(load().moe_cold_forward_host(C.byref(shape), _ptr(host_bank), _ptr(x), int(M),
                                        _ptr(topk_ids), _ptr(topk_w), _ptr(expert_to_slot),
                                        _ptr(y_cold), int(n_threads)), "moe_cold_forward_host")


class HybridStaging:
    """Pinned host buffers, a device buffer and two events for moe_layer_forward_hybrid."""

    def __init__(self, shape, max_M, device="cuda"):
        import torch
        H, k = shape.hidden, shape.top_k
        self.x = torch.zeros((max_M, H), dtype=torch.int16, pin_memory=True)
        self.ids = torch.zeros((max_M, k), dtype=torch.int32, pin_memory=True)
        self.w = torch.zeros((max_M, k), dtype=torch.float32, pin_memory=True)
        self.y_cold = torch.zeros((max_M, H), dtype=torch.float32, pin_memory=True)
        self.y_cold_dev = torch.zeros((max_M, H), dtype=torch.float32, device=device)
        self.routed = event_create(timing=False)
        self.added = event_create(timing=False)
        self.s = moe_hybrid_staging(max_M, _ptr(self.x), _ptr(self.ids), _ptr(self.w),
                                    _ptr(self.y_cold), _ptr(self.y_cold_dev), self.routed,
                                    self.added, 0)

    def close(self):
        if self.routed:
            event_synchronize(self.added) if self.s.pending else None
            event_destroy(self.routed)
            event_destroy(self.added)
            self.routed = self.added = None


def moe_layer_forward_hybrid(shape, x, M, w_router, router_bias, expert_to_slot,
                             expert_to_slot_host, slots, host_bank, topk_ids, topk_w, y,
                             staging: HybridStaging, ws, n_threads=0, stream=None):
    """The layer with hot experts on the GPU and cold routes on the host cores (y = full output)."""
    _check(load().moe_layer_forward_hybrid(C.byref(shape), _ptr(x), int(M), _ptr(w_router),
                                           _ptr(router_bias), _ptr(expert_to_slot),
                                           _ptr(expert_to_slot_host), _ptr(slots), _ptr(host_bank),
                                           _ptr(topk_ids), _ptr(topk_w), _ptr(y),
                                           C.byref(staging.s), int(n_threads), _ptr(ws),
                                           _nbytes(ws), _stream(stream)),
           "moe_layer_forward_hybrid")


def moe_hbm_read_probe(src, nbytes, sink, stream=None):
    _check(load().moe_hbm_read_probe(_ptr(src), int(nbytes), _ptr(sink), _stream(stream)),
           "moe_hbm_read_probe")


def moe_residual_bf16(x, y, out, n, stream=None):
    _check(load().moe_residual_bf16(_ptr(x), _ptr(y), _ptr(out), int(n), _stream(stream)),
           "moe_residual_bf16")


def moe_slot_refill(shape, slots, host_bank, experts, slot_ids, copy_stream=None,
                    wait_before=None, done=None):
    ex = np.ascontiguousarray(experts, dtype=np.int32)
    sl = np.ascontiguousarray(slot_ids, dtype=np.int32)
    if ex.shape != sl.shape:
        raise ValueError("experts and slot_ids differ in length")
    _check(load().moe_slot_refill(C.byref(shape), _ptr(slots), _ptr(host_bank), _ptr(ex), _ptr(sl),
                                  int(ex.size), _stream(copy_stream), wait_before, done),
           "moe_slot_refill")


class MoeCache:
    """Owns one moe_cache object (host-only policy state for one layer)."""

    def __init__(self, shape: moe_shape, policy=MOE_POLICY_LRU, max_refills_per_step=2,
                 lag_steps=1, max_pending=2, decay_period=64, initial_slot_expert=None):
        self.shape = shape
        cfg = moe_cache_config(policy, max_refills_per_step, lag_steps, max_pending, decay_period)
        init = None
        if initial_slot_expert is not None:
            init = np.ascontiguousarray(initial_slot_expert, dtype=np.int32)
            if init.size != shape.n_slots:
                raise ValueError("initial_slot_expert must have n_slots entries")
        h = _P()
        _check(load().moe_cache_create(C.byref(shape), C.byref(cfg), _ptr(init), C.byref(h)),
               "moe_cache_create")
        self._h = h
        self._plan = (moe_refill * max(1, max_refills_per_step))()
        self._map = np.empty(shape.n_experts, dtype=np.int32)

    def moe_cache_policy_step(self, step: int, topk_ids=None):
        """Returns (expert_to_slot int32 [E], [(expert, slot, evicted, visible_step)], stats dict)."""
        ids = None if topk_ids is None else np.ascontiguousarray(topk_ids, dtype=np.int32)
        M = 0 if ids is None else ids.size // self.shape.top_k
        n = _I32(0)
        st = moe_cache_stats()
        _check(load().moe_cache_policy_step(self._h, int(step), _ptr(ids), M, C.addressof(self._plan),
                                            C.byref(n), _ptr(self._map), C.byref(st)),
               "moe_cache_policy_step")
        plan = [(p.expert, p.slot, p.evicted, p.visible_step) for p in self._plan[: n.value]]
        stats = {f: getattr(st, f) for f, _ in moe_cache_stats._fields_}
        return self._map.copy(), plan, stats

    def moe_cache_save(self) -> np.ndarray:
        """The cache's whole state as bytes (moe_cache_save)."""
        n = _SZ(0)
        _check(load().moe_cache_state_bytes(self._h, C.byref(n)), "moe_cache_state_bytes")
        buf = np.zeros(n.value, dtype=np.uint8)
        _check(load().moe_cache_save(self._h, _ptr(buf), buf.nbytes), "moe_cache_save")
        return buf

    def moe_cache_restore(self, state: np.ndarray):
        """Loads a saved state (moe_cache_restore); the saved configuration comes with it."""
        buf = np.ascontiguousarray(state, dtype=np.uint8)
        _check(load().moe_cache_restore(self._h, _ptr(buf), buf.nbytes), "moe_cache_restore")
        # the plan buffer holds the restored configuration's refills per step (the header's
        # configuration follows magic, version, E, S, k)
        cfg = moe_cache_config.from_buffer_copy(buf[20:20 + C.sizeof(moe_cache_config)].tobytes())
        self._plan = (moe_refill * max(1, cfg.max_refills_per_step))()

    def close(self):
        if self._h:
            load().moe_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class PrefillStaging:
    """Staging slots, count / map buffers, a copy stream and events for moe_layer_forward_staged."""

    def __init__(self, shape, max_M, n_slots, device="cuda"):
        import torch
        E, H = shape.n_experts, shape.hidden
        img = moe_expert_image_bytes(shape)
        self.slots = torch.zeros((n_slots, img), dtype=torch.uint8, device=device)
        self.counts_dev = torch.zeros(E, dtype=torch.int32, device=device)
        self.counts_host = torch.zeros(E, dtype=torch.int32, pin_memory=True)
        self.maps_dev = torch.zeros((2, E), dtype=torch.int32, device=device)
        self.maps_host = torch.zeros((2, E), dtype=torch.int32, pin_memory=True)
        self.y_pass = torch.zeros((max_M, H), dtype=torch.float32, device=device)
        self.copy_stream = torch.cuda.Stream()
        self.events = [event_create() for _ in range(5)]
        ev = self.events
        self.s = moe_prefill_staging(max_M, n_slots, _ptr(self.slots), _ptr(self.counts_dev),
                                     _ptr(self.counts_host), _ptr(self.maps_dev),
                                     _ptr(self.maps_host), _ptr(self.y_pass),
                                     self.copy_stream.cuda_stream, ev[0],
                                     (C.c_void_p * 2)(ev[1], ev[2]), (C.c_void_p * 2)(ev[3], ev[4]),
                                     (C.c_int32 * 2)(0, 0))

    def close(self):
        import torch
        torch.cuda.synchronize()
        for e in self.events:
            event_destroy(e)
        self.events = []


def moe_layer_forward_staged(shape, x, M, w_router, router_bias, host_bank, topk_ids, topk_w, y,
                             staging: PrefillStaging, ws, stream=None):
    """The layer with its touched experts staged from pinned host memory; returns (touched, passes)."""
    nt, npass = _I32(0), _I32(0)
    _check(load().moe_layer_forward_staged(C.byref(shape), _ptr(x), int(M), _ptr(w_router),
                                           _ptr(router_bias), _ptr(host_bank), _ptr(topk_ids),
                                           _ptr(topk_w), _ptr(y), C.byref(staging.s), _ptr(ws),
                                           _nbytes(ws), _stream(stream), C.byref(nt), C.byref(npass)),
           "moe_layer_forward_staged")
    return nt.value, npass.value


class DeviceCache:
    """One layer's GPU-resident slot cache: its device state (torch uint8 tensor) and the
    entry points that act on it."""

    def __init__(self, shape: moe_shape, policy=MOE_POLICY_LRU, max_refills_per_step=2,
                 lag_steps=1, max_pending=2, decay_period=64, initial_slot_expert=None,
                 first_step=0, stream=None, device="cuda"):
        import torch
        self.shape = shape
        n = _SZ(0)
        _check(load().moe_device_cache_size(C.byref(shape), C.byref(n)), "moe_device_cache_size")
        self.state = torch.zeros(n.value, dtype=torch.uint8, device=device)
        cfg = moe_cache_config(policy, max_refills_per_step, lag_steps, max_pending, decay_period)
        init = None
        if initial_slot_expert is not None:
            init = np.ascontiguousarray(initial_slot_expert, dtype=np.int32)
        _check(load().moe_device_cache_init(C.byref(shape), C.byref(cfg), _ptr(init),
                                            int(first_step), _ptr(self.state), n.value,
                                            _stream(stream)), "moe_device_cache_init")

    def step(self, observed_ids, n_observed, expert_to_slot, plan, n_plan, stream=None):
        """Enqueue one policy step.  plan: device buffer of >= R moe_refill records (24 bytes
        each); n_plan: one int32 on the device."""
        _check(load().moe_device_cache_step(C.byref(self.shape), _ptr(self.state),
                                            _nbytes(self.state), _ptr(observed_ids),
                                            int(n_observed), _ptr(expert_to_slot), _ptr(plan),
                                            _ptr(n_plan), _stream(stream)), "moe_device_cache_step")

    def copy(self, n_plan, plan, host_bank, slots, stream=None):
        _check(load().moe_device_cache_copy(C.byref(self.shape), _ptr(n_plan), _ptr(plan),
                                            _ptr(host_bank), _ptr(slots), _stream(stream)),
               "moe_device_cache_copy")

    def stats(self, stream=None):
        import torch
        out = torch.zeros(5, dtype=torch.int64, device=self.state.device)
        _check(load().moe_device_cache_stats(C.byref(self.shape), _ptr(self.state),
                                             _nbytes(self.state), _ptr(out), _stream(stream)),
               "moe_device_cache_stats")
        torch.cuda.synchronize()
        return dict(zip([f for f, _ in moe_cache_stats._fields_], out.cpu().tolist()))


REFILL_RECORD_BYTES = C.sizeof(moe_refill)


# ---------------------------------------------------------------------------------------------
# HIP events (plumbing for refill ordering and kernel timing)
# ---------------------------------------------------------------------------------------------
_hip = None


def hip():
    global _hip
    if _hip is None:
        _hip = C.CDLL("libamdhip64.so")
        _hip.hipEventCreateWithFlags.argtypes = [C.POINTER(_P), C.c_uint]
        _hip.hipEventRecord.argtypes = [_P, _P]
        _hip.hipEventSynchronize.argtypes = [_P]
        _hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), _P, _P]
        _hip.hipEventDestroy.argtypes = [_P]
        _hip.hipStreamWaitEvent.argtypes = [_P, _P, C.c_uint]
        _hip.hipEventQuery.argtypes = [_P]
    return _hip


def _hipcheck(err, what):
    if err != 0:
        raise RuntimeError(f"{what} failed with HIP error {err}")


HIP_EVENT_DISABLE_TIMING = 0x2
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


def event_create(timing: bool = False, system_fence: bool = True) -> int:
    """A HIP event; timing=False disables timing, system_fence=False drops the system-scope
    fence of its records (cheaper, for marks that only time GPU work)."""
    flags = (0 if timing else HIP_EVENT_DISABLE_TIMING) | (0 if system_fence else HIP_EVENT_DISABLE_SYSTEM_FENCE)
    ev = _P()
    _hipcheck(hip().hipEventCreateWithFlags(C.byref(ev), flags), "hipEventCreateWithFlags")
    return ev.value


def event_record(ev: int, stream=None):
    _hipcheck(hip().hipEventRecord(ev, _stream(stream)), "hipEventRecord")


def event_synchronize(ev: int):
    _hipcheck(hip().hipEventSynchronize(ev), "hipEventSynchronize")


def event_done(ev: int) -> bool:
    return hip().hipEventQuery(ev) == 0


def event_elapsed_ms(start: int, stop: int) -> float:
    ms = C.c_float(0)
    _hipcheck(hip().hipEventElapsedTime(C.byref(ms), start, stop), "hipEventElapsedTime")
    return ms.value


def event_destroy(ev: int):
    hip().hipEventDestroy(ev)


def stream_wait_event(stream, ev: int):
    _hipcheck(hip().hipStreamWaitEvent(_stream(stream), ev, 0), "hipStreamWaitEvent")
