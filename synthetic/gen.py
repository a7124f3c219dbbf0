"""Seeded generators for the routed-MoE workloads.

Every random draw comes from numpy's PCG64 seeded with
``SeedSequence([workload_id, stream, layer, index])`` so that any expert, router, activation
batch or prior can be regenerated on its own, in any order, on any machine.

Streams: 0 = expert weights, 1 = router weights, 2 = activations, 3 = popularity
permutation, 4 = warm-up activations.

Recipe (the pages give no weights or prompts; these stand in for them at the pages' shapes):
  * expert weights: fp32 N(0, 0.02), then MXFP4-encoded per 32-element block along the input
    dimension (``quantize_mxfp4``); the other expert formats encode the same draw (bf16
    rounding, ``quantize_fp8_block``, ``quantize_nvfp4``);
  * router: fp32 N(0, 0.02) rounded to bf16;
  * activations: fp32 N(0, 1) rounded to bf16;
  * popularity prior: a seeded permutation gives each expert a rank r in 1..E and its logit
    bias is -s*ln(r) (the log of an unnormalised Zipf(s) pmf).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

STREAM_WEIGHTS = 0
STREAM_ROUTER = 1
STREAM_ACT = 2
STREAM_PRIOR = 3
STREAM_WARMUP = 4

WEIGHT_STD = 0.02
ROUTER_STD = 0.02


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int  # seed namespace
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    tokens: tuple  # the M values this workload runs at
    n_slots: int
    zipf_s: float | None = None
    steps: int = 1
    layers: int = 1
    drift_period: int = 0  # steps between cyclic shifts of the popularity ranks (0 = none)


WORKLOADS = {
    # Tiny layer: every expert resident, no prior.
    "tiny": Workload("tiny", 1, 256, 512, 8, 2, (4,), 8),
    # GPT-OSS-20B-shaped layer, M=1 decode over 256 steps, Zipf(1.1) prior, all resident.
    "gptoss20b_decode": Workload("gptoss20b_decode", 2, 2880, 2880, 32, 4, (1,), 32,
                                 zipf_s=1.1, steps=256),
    # Same layer with only 8 GPU slots, LRU refills, drifting popularity.
    "gptoss20b_8slots": Workload("gptoss20b_8slots", 3, 2880, 2880, 32, 4, (1,), 8,
                                 zipf_s=1.1, steps=256, drift_period=32),
    # Fine-grained E=512 layer stack, speculative-verify token counts, 256 of 512 resident.
    "e512_verify_stack": Workload("e512_verify_stack", 4, 2048, 512, 512, 10, (1, 4, 8), 256,
                                  zipf_s=1.0, steps=256, layers=48),
    # Batched / prefill E=512 layer, every expert resident.
    "e512_prefill": Workload("e512_prefill", 5, 2048, 512, 512, 10, (512,), 512, zipf_s=1.0),
}


def _rng(wid: int, stream: int, layer: int = 0, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([wid, stream, layer, index])))


def bf16_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    out = ((bits + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def quantize_mxfp4(w: np.ndarray):
    """Encode an fp32 matrix [N, K] (K % 32 == 0) as MXFP4 bytes.

    Returns ``(codes uint8 [N, K/2], scales uint8 [N, K/32])``.  Per 32-element block along K:
    X = clamp(floor(log2(amax)) - 2 + 127, 0, 254) (127 when the block is all zero); each
    element w / 2^(X-127) is rounded to the nearest E2M1 magnitude {0,.5,1,1.5,2,3,4,6}
    (ties to the even code, saturating at 6) and its sign goes to bit 3.  Element 2c sits in
    the low nibble of byte c, element 2c+1 in the high nibble.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    blk = w.reshape(n, k // 32, 32)
    amax = np.abs(blk).max(axis=2)
    _, e = np.frexp(amax)  # amax = m * 2**e with m in [0.5, 1)  ->  floor(log2 amax) = e - 1
    x = np.clip(e.astype(np.int32) - 1 - 2 + 127, 0, 254)
    x = np.where(amax == 0, 127, x).astype(np.int32)
    v = np.ldexp(blk, (127 - x)[..., None]).astype(np.float32)
    code = _e2m1_codes(v).reshape(n, k)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return np.ascontiguousarray(packed), np.ascontiguousarray(x.astype(np.uint8))


def _e2m1_codes(v: np.ndarray) -> np.ndarray:
    """4-bit E2M1 codes of values already divided by their scale: nearest magnitude of
    {0, .5, 1, 1.5, 2, 3, 4, 6} (ties to the even code, saturating at 6), sign in bit 3."""
    a = np.abs(v)
    # index of the nearest magnitude: '>' where a tie goes down to the even code, '>=' where it
    # goes up to the even code
    mag = (a > 0.25).astype(np.uint8)
    mag += a >= 0.75
    mag += a > 1.25
    mag += a >= 1.75
    mag += a > 2.5
    mag += a >= 3.5
    mag += a > 5.0
    return mag | (((v < 0) & (mag > 0)).astype(np.uint8) << 3)


def encode_e4m3(v: np.ndarray):
    """OCP E4M3 codes of fp32 values with |v| <= 448, rounded to nearest even.

    Returns ``(codes uint8, values float64)``: the values the codes stand for.  A magnitude a
    in the binade [2^e, 2^(e+1)) (e >= -6; below 2^-6 the subnormals share the step of that
    binade) is rounded to a multiple of 2^(e-3); a result of 16 steps moves to the next binade.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > 448):
        raise ValueError("E4M3 holds magnitudes up to 448")
    _, ex = np.frexp(a)
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    e = np.where(a == 0, -6, e)
    m = np.rint(np.ldexp(a, (3 - e).astype(np.int64)))  # 0 .. 16, halves to even
    up = m >= 16
    e = np.where(up, e + 1, e)
    m = np.where(up, 8, m).astype(np.int64)
    code = np.where((e == -6) & (m < 8), m, ((e + 7) << 3) | (m - 8))
    value = np.ldexp(m.astype(np.float64), (e - 3).astype(np.int64))
    neg = (v < 0) & (code > 0)
    code = code | (neg.astype(np.int64) << 7)
    return code.astype(np.uint8), np.where(neg, -value, value)


def quantize_fp8_block(w: np.ndarray):
    """Encode an fp32 matrix [N, K] as block FP8: E4M3 codes [N, K] and fp32 scales
    [ceil(N/128), ceil(K/128)], the scale of a 128 x 128 block being amax / 448 (1 when zero)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    nb, kb = (n + 127) // 128, (k + 127) // 128
    scales = np.ones((nb, kb), dtype=np.float32)
    codes = np.empty((n, k), dtype=np.uint8)
    for bi in range(nb):
        for bj in range(kb):
            blk = w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            amax = float(np.abs(blk).max())
            s = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
            scales[bi, bj] = s
            q = np.clip(blk.astype(np.float64) / float(s), -448.0, 448.0)
            codes[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128] = encode_e4m3(q)[0]
    return codes, scales


def quantize_nvfp4(w: np.ndarray):
    """Encode an fp32 matrix [N, K] (K % 16 == 0) as NVFP4.

    Returns ``(codes uint8 [N, K/2], scales uint8 [N, K/16], global_scale float)``: g =
    amax(matrix) / (6 * 448); each 16-element block gets the E4M3 code of amax(block) / 6 / g;
    each element w / (block scale value * g) is rounded to E2M1 (element 2c in the low nibble of
    byte c).
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    if k % 16:
        raise ValueError("K must be a multiple of 16")
    amax = float(np.abs(w).max())
    g = float(np.float32(amax / (6.0 * 448.0))) if amax > 0 else 1.0
    blk = w.reshape(n, k // 16, 16).astype(np.float64)
    bmax = np.abs(blk).max(axis=2)
    sc, sval = encode_e4m3(np.minimum(bmax / 6.0 / g, 448.0))
    denom = sval * g
    v = np.where(denom[..., None] > 0, blk / np.where(denom > 0, denom, 1.0)[..., None], 0.0)
    code = _e2m1_codes(v).reshape(n, k)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return np.ascontiguousarray(packed), np.ascontiguousarray(sc), g


def expert_canonical(wl: Workload, layer: int, expert: int, fmt: str = "mxfp4") -> dict:
    """One expert's weights in canonical row-major layout, encoded in ``fmt``.

    gate, up: [inter, hidden]; down: [hidden, inter] (rows = outputs, blocks along inputs).
    The fp32 weights are the same draw for every format.  Keys: "<m>_codes" (elements: bf16
    bits uint16 for "bf16", else uint8 codes) and "<m>_scales" (E8M0 bytes for "mxfp4", fp32
    block scales for "fp8_block", E4M3 bytes for "nvfp4", whose fp32 matrix scale is
    "<m>_global"); the dict carries "format" for every format but MXFP4.
    """
    rng = _rng(wl.wid, STREAM_WEIGHTS, layer, expert)
    h, i = wl.hidden, wl.inter
    out = {} if fmt == "mxfp4" else {"format": fmt}
    for name, shape in (("gate", (i, h)), ("up", (i, h)), ("down", (h, i))):
        w = rng.standard_normal(shape, dtype=np.float32) * np.float32(WEIGHT_STD)
        if fmt == "mxfp4":
            out[name + "_codes"], out[name + "_scales"] = quantize_mxfp4(w)
        elif fmt == "bf16":
            out[name + "_codes"] = bf16_from_f32(w)
        elif fmt == "fp8_block":
            out[name + "_codes"], out[name + "_scales"] = quantize_fp8_block(w)
        elif fmt == "nvfp4":
            out[name + "_codes"], out[name + "_scales"], out[name + "_global"] = quantize_nvfp4(w)
        else:
            raise ValueError(f"unknown format {fmt!r}")
    return out


def experts_canonical(wl: Workload, layer: int, experts, threads: int | None = None,
                      fmt: str = "mxfp4") -> list:
    """Generate several experts in parallel threads (numpy releases the GIL in bulk ops)."""
    experts = list(experts)
    threads = threads or min(16, os.cpu_count() or 1, max(1, len(experts)))
    with ThreadPoolExecutor(max_workers=threads) as pool:
        return list(pool.map(lambda e: expert_canonical(wl, layer, e, fmt), experts))


def router_weights(wl: Workload, layer: int = 0) -> np.ndarray:
    """Router matrix W_r [E, hidden] as bf16 bits."""
    rng = _rng(wl.wid, STREAM_ROUTER, layer, 0)
    w = rng.standard_normal((wl.n_experts, wl.hidden), dtype=np.float32) * np.float32(ROUTER_STD)
    return bf16_from_f32(w)


def activations(wl: Workload, M: int, step: int, layer: int = 0, warmup: bool = False) -> np.ndarray:
    """Token activations x [M, hidden] as bf16 bits for one step."""
    rng = _rng(wl.wid, STREAM_WARMUP if warmup else STREAM_ACT, layer, step * 4096 + M)
    return bf16_from_f32(rng.standard_normal((M, wl.hidden), dtype=np.float32))


def zipf_ranks(wl: Workload, layer: int = 0, shift: int = 0) -> np.ndarray:
    """Popularity rank (1 = most popular) of every expert.

    A seeded permutation assigns ranks; ``shift`` applies the drift: every shift moves each
    rank one place down cyclically (rank E becomes 1, every other rank r becomes r+1).
    """
    perm = _rng(wl.wid, STREAM_PRIOR, layer, 0).permutation(wl.n_experts)
    ranks = np.empty(wl.n_experts, dtype=np.int64)
    ranks[perm] = np.arange(1, wl.n_experts + 1)
    return (ranks - 1 + shift) % wl.n_experts + 1


def zipf_bias(wl: Workload, layer: int = 0, shift: int = 0) -> np.ndarray:
    """Router logit bias b_e = -s * ln(rank_e) as float32 (zeros when the workload has no prior)."""
    if wl.zipf_s is None:
        return np.zeros(wl.n_experts, dtype=np.float32)
    r = zipf_ranks(wl, layer, shift).astype(np.float64)
    return (-wl.zipf_s * np.log(r)).astype(np.float32)


def drift_shift(wl: Workload, step: int) -> int:
    """Number of cyclic rank shifts in force at ``step``."""
    return step // wl.drift_period if wl.drift_period else 0
