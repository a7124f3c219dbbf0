"""Pins of the oracle's MXFP4 decode against the format definition (golden table) and torch.

The golden table (tests/golden/mxfp4_element_values.txt) writes out the OCP MX v1.0 E2M1 and
E8M0 values; torch's float8_e8m0fnu dtype is an independent library decoder for the scales.
"""
import os

import numpy as np
import pytest
import torch

from oracle import mxfp4
from oracle.layer import bf16_to_f64, f64_to_bf16_rne

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_element_values.txt")


def _golden():
    e2m1, e8m0 = {}, {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        kind, code, val = line.split()
        (e2m1 if kind == "e2m1" else e8m0)[int(code, 16)] = float(val)
    return e2m1, e8m0


def _same(a, b):
    return (np.isnan(a) and np.isnan(b)) or (a == b and np.signbit(a) == np.signbit(b))


def test_e2m1_all_codes_match_table():
    e2m1, _ = _golden()
    assert sorted(e2m1) == list(range(16))
    for code, val in e2m1.items():
        assert _same(mxfp4.e2m1_value(code), val), code


def test_e8m0_matches_table_and_torch():
    _, e8m0 = _golden()
    for x, val in e8m0.items():
        assert _same(mxfp4.e8m0_value(x), val), x
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for x in range(256):
        assert _same(mxfp4.e8m0_value(x), float(ref[x])), x


@pytest.mark.parametrize("scale_byte", [1, 120, 127, 128, 134, 254, 255])
def test_hand_built_block_nibble_order(scale_byte):
    e2m1, e8m0 = _golden()
    # byte c holds element 2c (low nibble) and 2c+1 (high nibble), distinct codes per position
    lo = np.arange(16) % 16
    hi = (np.arange(16) + 5) % 16
    codes = (lo | (hi << 4)).astype(np.uint8)[None, :]
    scales = np.array([[scale_byte]], dtype=np.uint8)
    out = mxfp4.dequantize(codes, scales)[0]
    s = e8m0[scale_byte] if scale_byte in e8m0 else 2.0 ** (scale_byte - 127)
    for c in range(16):
        assert _same(out[2 * c], e2m1[lo[c]] * s), (c, "low")
        assert _same(out[2 * c + 1], e2m1[hi[c]] * s), (c, "high")


def test_block_scale_indexing_rows_and_blocks():
    # 3 rows x 3 blocks; every element code 0x2 (1.0); scale differs per (row, block)
    codes = np.full((3, 48), 0x22, dtype=np.uint8)
    scales = np.array([[120, 121, 122], [130, 131, 132], [100, 101, 102]], dtype=np.uint8)
    out = mxfp4.dequantize(codes, scales)
    for r in range(3):
        for b in range(3):
            assert np.all(out[r, 32 * b: 32 * b + 32] == 2.0 ** (int(scales[r, b]) - 127))


def test_dequant_exact_in_bf16():
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 256, size=(8, 64), dtype=np.uint8)
    scales = rng.integers(100, 150, size=(8, 4), dtype=np.uint8)
    v = mxfp4.dequantize(codes, scales)
    back = bf16_to_f64(f64_to_bf16_rne(v))
    assert np.array_equal(back, v)
