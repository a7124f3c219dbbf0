"""The input recipe: the MXFP4 encoder's rounding rule and bound, determinism of the generators."""
import numpy as np

import synthetic
from oracle import mxfp4

E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)


def test_encoder_scale_rule_at_powers_of_two():
    for j in range(-20, 10):
        w = np.zeros((1, 32), dtype=np.float32)
        w[0, 5] = 2.0 ** j
        codes, scales = synthetic.quantize_mxfp4(w)
        assert int(scales[0, 0]) == j - 2 + 127
        # the block maximum lands on E2M1 4.0 (code 6) exactly
        assert mxfp4.dequantize(codes, scales)[0, 5] == 2.0 ** j
    codes, scales = synthetic.quantize_mxfp4(np.zeros((2, 64), dtype=np.float32))
    assert np.all(scales == 127) and np.all(codes == 0)


def test_encoder_ties_go_to_even_codes():
    # scale 2^0 (amax in [4, 8)): element values on the midpoints between E2M1 magnitudes
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0], dtype=np.float32)
    expect = np.array([0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0])
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, :8] = mids
    w[0, 8:16] = -mids
    w[0, 31] = 4.0
    codes, scales = synthetic.quantize_mxfp4(w)
    assert scales[0, 0] == 127
    v = mxfp4.dequantize(codes, scales)[0]
    assert np.array_equal(v[:8], expect)
    assert np.array_equal(v[8:16], -expect)


def test_encoder_round_trip_bound():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    codes, scales = synthetic.quantize_mxfp4(w)
    q = mxfp4.dequantize(codes, scales)
    s = np.repeat(2.0 ** (scales.astype(np.float64) - 127), 32, axis=1)
    v = np.abs(w.astype(np.float64)) / s
    # half the local E2M1 spacing: 0.25 below 2, 0.5 in [2, 4), 1 at and above 4 (saturation at 6)
    half = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    ok = v <= 6
    assert np.all((np.abs(w - q) <= half * s + 1e-30)[ok])
    # above 6 (possible up to 8, since amax / scale lies in [4, 8)) the encoder saturates
    assert np.all((np.abs(q) == 6 * s)[~ok]) and (~ok).any()
    assert np.all(np.sign(q[q != 0]) == np.sign(w[q != 0]))


def test_generators_are_deterministic_and_shaped():
    wl = synthetic.WORKLOADS["gptoss20b_decode"]
    a = synthetic.router_weights(wl)
    b = synthetic.router_weights(wl)
    assert a.shape == (32, 2880) and a.dtype == np.uint16 and np.array_equal(a, b)
    x = synthetic.activations(wl, 1, 17)
    assert x.shape == (1, 2880) and np.array_equal(x, synthetic.activations(wl, 1, 17))
    assert not np.array_equal(x, synthetic.activations(wl, 1, 18))
    r = synthetic.zipf_ranks(wl)
    assert sorted(r.tolist()) == list(range(1, 33))
    r1 = synthetic.zipf_ranks(wl, shift=1)
    assert np.array_equal(r1, np.where(r == 32, 1, r + 1))
    bias = synthetic.zipf_bias(wl)
    assert np.allclose(bias, -1.1 * np.log(r), rtol=1e-6)
    tiny = synthetic.WORKLOADS["tiny"]
    ex = synthetic.expert_canonical(tiny, 0, 3)
    assert ex["gate_codes"].shape == (512, 128) and ex["gate_scales"].shape == (512, 8)
    assert ex["down_codes"].shape == (256, 256) and ex["down_scales"].shape == (256, 16)
