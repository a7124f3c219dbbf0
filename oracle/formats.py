"""Decode of the expert formats other than MXFP4, written from their published definitions.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU baseline use it.

MoE expert offload (xinfer docs), "Supported": unquantised bf16, block FP8 and NVFP4 experts
go through the same generic slot path as MXFP4.  The page names the formats but does not define
them; the definitions followed here are the usual published ones (readings):

  bf16       the upper 16 bits of an IEEE-754 binary32 value.
  E4M3       OCP 8-bit floating point (OFP8) E4M3: bit 7 sign, bits 6..3 exponent e (bias 7),
             bits 2..0 mantissa m.  e = 0: subnormal m/8 * 2^-6; e > 0: 2^(e-7) * (1 + m/8);
             S.1111.111 is NaN; there are no infinities (largest finite value 448).
  FP8 block  W[n, k] = E4M3(c[n, k]) * s[n // 128, k // 128], with one fp32 scale s per
             128 x 128 block of the [N, K] matrix (partial blocks at the right and bottom edge).
  NVFP4      W[n, k] = E2M1(c[n, k]) * E4M3(s[n, k // 16]) * g: FP4 E2M1 elements (as in MXFP4,
             element 2c in the low nibble of byte c), one E4M3 scale per 16 elements along K and
             one fp32 scale g of the whole matrix.

Every decode is exact in float64 (the products have at most 3 + 4 + 24 significant bits).
"""
from __future__ import annotations

import numpy as np

from . import mxfp4

FORMATS = ("mxfp4", "bf16", "fp8_block", "nvfp4")


def e4m3_value(code: int) -> float:
    """Value of one E4M3 byte, from its sign / exponent / mantissa fields."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return sign * mag


_E4M3 = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def bf16_values(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def dequantize_fp8_block(codes, scales) -> np.ndarray:
    """codes uint8 [N, K] (E4M3), scales float32 [ceil(N/128), ceil(K/128)] -> float64 [N, K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.float32).astype(np.float64)
    n, k = codes.shape
    nb, kb = (n + 127) // 128, (k + 127) // 128
    if scales.shape != (nb, kb):
        raise ValueError(f"scales shape {scales.shape} != {(nb, kb)}")
    rows = np.arange(n) // 128
    cols = np.arange(k) // 128
    return _E4M3[codes] * scales[rows[:, None], cols[None, :]]


def dequantize_nvfp4(codes, scales, global_scale) -> np.ndarray:
    """codes uint8 [N, K/2] (E2M1 pairs), scales uint8 [N, K/16] (E4M3), global fp32 -> [N, K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    n, half = codes.shape
    k = 2 * half
    if scales.shape != (n, k // 16):
        raise ValueError(f"scales shape {scales.shape} != {(n, k // 16)}")
    elem = np.empty((n, k), dtype=np.uint8)
    elem[:, 0::2] = codes & 0x0F
    elem[:, 1::2] = codes >> 4
    table = np.array([mxfp4.e2m1_value(c) for c in range(16)], dtype=np.float64)
    g = float(np.float32(global_scale))
    block = _E4M3[scales]  # [N, K/16]
    return table[elem] * np.repeat(block, 16, axis=1) * g


def dequantize_matrix(expert: dict, name: str) -> np.ndarray:
    """One matrix ("gate", "up" or "down") of an expert dict in its format, as float64."""
    fmt = expert.get("format", "mxfp4")
    if fmt == "mxfp4":
        return mxfp4.dequantize(expert[name + "_codes"], expert[name + "_scales"])
    if fmt == "bf16":
        return bf16_values(expert[name + "_codes"])
    if fmt == "fp8_block":
        return dequantize_fp8_block(expert[name + "_codes"], expert[name + "_scales"])
    if fmt == "nvfp4":
        return dequantize_nvfp4(expert[name + "_codes"], expert[name + "_scales"],
                                expert[name + "_global"])
    raise ValueError(f"unknown expert format {fmt!r}")
