"""Pins of the oracle's decode of the other expert formats (bf16, block FP8, NVFP4).

Each pin ties the decode to something other than itself: the OCP E4M3 values written out in
tests/golden/e4m3_values.txt, torch's float8_e4m3fn and bfloat16 dtypes (independent library
decoders), hand-built matrices whose expected values follow from the layout definitions alone
(so that a transposed or shifted scale index fails), the error bounds of the synthetic encoders
(written separately from the decoders), and a cross-format invariant: the same values held as
MXFP4 (whose decode is pinned on its own), bf16 and NVFP4 give the same layer output.
"""
import os

import numpy as np
import pytest
import torch

import synthetic
from oracle import formats, mxfp4
from oracle import layer as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_values.txt")


def _same(a, b):
    return (np.isnan(a) and np.isnan(b)) or (a == b and np.signbit(a) == np.signbit(b))


def test_e4m3_matches_golden_values():
    n = 0
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        assert _same(formats.e4m3_value(int(code, 16)), float(val)), code
        n += 1
    assert n >= 20


def test_e4m3_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        assert _same(formats.e4m3_value(c), ref[c]), hex(c)


def test_bf16_values_match_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 1 << 16, 4096, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = formats.bf16_values(bits)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(got[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_fp8_block_scale_index_follows_row_and_column_blocks():
    # 130 x 260: a 2 x 3 grid of 128 x 128 blocks with ragged right and bottom edges
    n, k = 130, 260
    codes = np.full((n, k), 0x38, dtype=np.uint8)  # every element 1.0
    scales = (np.arange(6, dtype=np.float32).reshape(2, 3) + 1) * np.float32(0.25)
    w = formats.dequantize_fp8_block(codes, scales)
    for r, c in [(0, 0), (127, 127), (128, 0), (129, 259), (5, 128), (5, 256), (128, 200)]:
        assert w[r, c] == scales[r // 128, c // 128], (r, c)
    # an element code times its block's scale
    codes[129, 257] = 0xC4  # -3.0
    assert formats.dequantize_fp8_block(codes, scales)[129, 257] == -3.0 * float(scales[1, 2])
    with pytest.raises(ValueError):
        formats.dequantize_fp8_block(codes, scales.T)


def test_nvfp4_nibble_order_block_scale_and_global():
    n, k = 3, 64
    codes = np.full((n, k // 2), 0x22, dtype=np.uint8)  # E2M1 code 2 = 1.0 in both nibbles
    codes[1, 0] = 0x52  # element 0: code 2 (1.0), element 1: code 5 (3.0)
    scales = np.full((n, k // 16), 0x38, dtype=np.uint8)  # 1.0
    scales[2, 3] = 0x40  # 2.0 for row 2, elements 48..63
    g = 0.5
    w = formats.dequantize_nvfp4(codes, scales, g)
    assert w[1, 0] == 0.5 and w[1, 1] == 1.5
    assert w[2, 47] == 0.5 and w[2, 48] == 1.0 and w[2, 63] == 1.0
    assert w[0, 63] == 0.5
    # the block scale is per 16 elements of a row, not per 32
    scales[0, 1] = 0x48  # 4.0 for row 0, elements 16..31
    w = formats.dequantize_nvfp4(codes, scales, g)
    assert w[0, 15] == 0.5 and w[0, 16] == 2.0 and w[0, 31] == 2.0 and w[0, 32] == 0.5


@pytest.mark.parametrize("shape", [(256, 512), (130, 96)])
def test_fp8_block_encoder_error_bound(shape):
    rng = np.random.default_rng(7)
    w = rng.standard_normal(shape).astype(np.float32) * np.float32(0.02)
    codes, scales = synthetic.quantize_fp8_block(w)
    dq = formats.dequantize_fp8_block(codes, scales)
    s = scales.astype(np.float64)[np.arange(shape[0])[:, None] // 128,
                                  np.arange(shape[1])[None, :] // 128]
    q = np.abs(w.astype(np.float64)) / s  # <= 448
    # E4M3 rounding: half a step, 2^-4 of the magnitude for normals, 2^-10 for subnormals
    bound = s * np.maximum(q * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(dq - w) <= bound)
    # the largest element of each block maps to 448 exactly
    assert np.isclose(np.abs(dq).max(), np.abs(w).max(), rtol=1e-6)


@pytest.mark.parametrize("shape", [(256, 512), (96, 160)])
def test_nvfp4_encoder_error_bound(shape):
    rng = np.random.default_rng(11)
    w = rng.standard_normal(shape).astype(np.float32) * np.float32(0.02)
    codes, scales, g = synthetic.quantize_nvfp4(w)
    dq = formats.dequantize_nvfp4(codes, scales, g)
    sv = np.repeat(np.array([formats.e4m3_value(c) for c in scales.reshape(-1)]).reshape(scales.shape),
                   16, axis=1) * g
    # E2M1 rounding: at most a quarter of the magnitude (or 0.25 units) of the scaled value, and
    # a little saturation past 6 where the block scale rounded down
    v = np.abs(w.astype(np.float64)) / sv
    bound = sv * np.maximum(np.maximum(0.25, v / 4), v - 6) * (1 + 1e-6)
    assert np.all(np.abs(dq - w) <= bound)
    assert np.max(np.abs(dq - w)) < 0.25 * np.abs(w).max()


def _mx_expert_as(fmt, mx: dict) -> dict:
    """The values of an MXFP4 expert, held exactly in another format (built from the MXFP4 bytes
    and torch's conversions; no oracle decode involved beyond mxfp4, pinned elsewhere)."""
    out = {"format": fmt}
    for name in ("gate", "up", "down"):
        c, s = mx[name + "_codes"], mx[name + "_scales"]
        if fmt == "bf16":
            vals = mxfp4.dequantize(c, s)  # E2M1 x 2^p: at most 2 significant bits, exact in bf16
            out[name + "_codes"] = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        elif fmt == "nvfp4":
            # the same nibbles; each 32-block's 2^(X-127) becomes two 16-block E4M3 scales of
            # 2^(X-127+14) under the matrix scale 2^-14
            p = s.astype(np.float64) - 127 + 14
            assert p.min() >= -9 and p.max() <= 8, "powers of two outside E4M3's exact range"
            e4 = torch.from_numpy(np.exp2(p)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            out[name + "_codes"] = c.copy()
            out[name + "_scales"] = np.repeat(e4, 2, axis=1)
            out[name + "_global"] = 2.0 ** -14
        else:
            raise ValueError(fmt)
    return out


@pytest.mark.parametrize("fmt", ["bf16", "nvfp4"])
def test_same_values_in_another_format_give_the_same_layer(fmt):
    wl = synthetic.WORKLOADS["tiny"]
    experts = [synthetic.expert_canonical(wl, 0, e) for e in range(wl.n_experts)]
    other = [_mx_expert_as(fmt, ex) for ex in experts]
    for a, b in zip(experts, other):
        for name in ("gate", "up", "down"):
            assert np.array_equal(formats.dequantize_matrix(a, name), formats.dequantize_matrix(b, name))
    x = synthetic.activations(wl, 4, 0)
    rng = np.random.default_rng(5)
    ids = np.stack([rng.choice(wl.n_experts, wl.top_k, replace=False) for _ in range(4)])
    w = rng.random((4, wl.top_k))
    r0 = O.layer_forward(x, ids, w, experts)
    r1 = O.layer_forward(x, ids, w, other)
    assert np.array_equal(r0["y_full"], r1["y_full"])
    assert np.array_equal(r0["h_bits"], r1["h_bits"])


def test_synthetic_formats_share_one_weight_draw():
    # every format encodes the same fp32 draw: their decoded matrices agree to within the
    # coarsest format's error (NVFP4), far below the weights' spread
    wl = synthetic.WORKLOADS["tiny"]
    dense = {f: O.dequantize_expert(synthetic.expert_canonical(wl, 0, 3, f))
             for f in formats.FORMATS}
    ref = dense["bf16"]["gate"]
    for f in formats.FORMATS:
        err = np.linalg.norm(dense[f]["gate"] - ref) / np.linalg.norm(ref)
        assert err < 0.15, (f, err)
    assert np.linalg.norm(dense["fp8_block"]["gate"] - ref) / np.linalg.norm(ref) < 0.05
