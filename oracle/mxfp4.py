"""MXFP4 decode, written from the format's public definition.

The pages run "native MXFP4" experts without a fused bf16 copy (tinyserve README, "How it
works", items 1-2; MoE expert offload (xinfer docs), "Supported") but never define the
encoding.  The definition followed here is the OCP Microscaling Formats (MX) Specification
v1.0: a block of 32 elements shares one E8M0 scale; each element is an FP4 E2M1 number.

  E2M1 (4 bits, exponent bias 1, no inf/NaN): bit 3 = sign, bits 2..1 = exponent e,
        bit 0 = mantissa m.  e = 0 is subnormal: 0.5*m;  e > 0: 2^(e-1) * (1 + 0.5*m).
  E8M0 (8 bits, bias 127, no sign/mantissa): 2^(X-127); X = 255 is NaN.

Storage convention of this project (a reading; the pages are silent): a matrix [N, K] is
row-major, blocks run along K, element 2c of a row sits in the low nibble of byte c and
element 2c+1 in the high nibble; scales are [N, K/32].
"""
from __future__ import annotations

import numpy as np


def e2m1_value(code: int) -> float:
    """Value of one 4-bit E2M1 code, from its sign/exponent/mantissa fields."""
    code = int(code) & 0xF
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return sign * mag


def e8m0_value(x: int) -> float:
    """Value of one E8M0 scale byte."""
    x = int(x) & 0xFF
    return float("nan") if x == 255 else 2.0 ** (x - 127)


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode an MXFP4 matrix: codes uint8 [N, K/2], scales uint8 [N, K/32] -> float64 [N, K].

    Exact in float64 (every product is a power of two times a 3-significant-bit value).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    n, half = codes.shape
    k = half * 2
    if scales.shape != (n, k // 32):
        raise ValueError(f"scales shape {scales.shape} does not match codes {codes.shape}")
    elem = np.empty((n, k), dtype=np.uint8)
    elem[:, 0::2] = codes & 0x0F
    elem[:, 1::2] = codes >> 4
    table = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
    scale_table = np.array([e8m0_value(x) for x in range(256)], dtype=np.float64)
    vals = table[elem].reshape(n, k // 32, 32)
    return (vals * scale_table[scales][..., None]).reshape(n, k)
