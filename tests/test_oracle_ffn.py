"""Pins of the oracle's expert FFN, combine and route buckets.

The FFN is checked against a brute-force evaluation on a tiny expert: decode through the golden
E2M1/E8M0 table, pure-Python exactly-rounded dot products (math.fsum), a bf16 rounding found by
searching the sorted list of all bf16 values, and math.exp for SiLU.  The combine is checked
through the hot + cold = full invariant, its edge cases and slot relabelling.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import synthetic
from oracle import layer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_element_values.txt")


def _table():
    t = {}
    for line in open(GOLDEN):
        if line.startswith("e2m1"):
            _, c, v = line.split()
            t[int(c, 16)] = float(v)
    return t


def _decode_bruteforce(codes, scales):
    t = _table()
    n, half = codes.shape
    out = [[0.0] * (2 * half) for _ in range(n)]
    for r in range(n):
        for c in range(half):
            s = 2.0 ** (int(scales[r, (2 * c) // 32]) - 127)
            out[r][2 * c] = t[int(codes[r, c]) & 0xF] * s
            out[r][2 * c + 1] = t[int(codes[r, c]) >> 4] * s
    return out


_BF16 = None


def _bf16_round_bruteforce(a: float) -> float:
    global _BF16
    if _BF16 is None:
        bits = np.arange(0, 0x7F80, dtype=np.uint32)  # all finite non-negative bf16 values
        _BF16 = (bits << 16).view(np.float32).astype(np.float64)
    mag = abs(a)
    i = int(np.searchsorted(_BF16, mag))
    if i < len(_BF16) and _BF16[i] == mag:
        r = mag
    else:
        lo, hi = _BF16[i - 1], _BF16[i]
        dl, dh = Fraction(mag) - Fraction(lo), Fraction(hi) - Fraction(mag)
        if dl < dh:
            r = lo
        elif dh < dl:
            r = hi
        else:  # tie: the even bit pattern (index parity == mantissa lsb parity)
            r = lo if (i - 1) % 2 == 0 else hi
    return math.copysign(r, a)


def _tiny_expert(seed, H=64, I=32):
    rng = np.random.default_rng(seed)
    ex = {}
    for name, shape in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        w = (rng.standard_normal(shape) * 0.3).astype(np.float32)
        ex[name + "_codes"], ex[name + "_scales"] = synthetic.quantize_mxfp4(w)
    return ex


@pytest.mark.parametrize("seed", [0, 1])
def test_expert_ffn_bruteforce(seed):
    H, I = 64, 32
    ex = _tiny_expert(seed, H, I)
    rng = np.random.default_rng(100 + seed)
    x_bits = synthetic.bf16_from_f32(rng.standard_normal((2, H)).astype(np.float32))
    x = layer.bf16_to_f64(x_bits)
    h_bits, d = layer.expert_ffn(x, layer.dequantize_expert(ex))
    G = _decode_bruteforce(ex["gate_codes"], ex["gate_scales"])
    U = _decode_bruteforce(ex["up_codes"], ex["up_scales"])
    D = _decode_bruteforce(ex["down_codes"], ex["down_scales"])
    for m in range(2):
        xs = [float(v) for v in x[m]]
        hs = []
        for i in range(I):
            g = math.fsum(G[i][c] * xs[c] for c in range(H))
            u = math.fsum(U[i][c] * xs[c] for c in range(H))
            a = g / (1.0 + math.exp(-g)) * u
            hs.append(_bf16_round_bruteforce(a))
        got_h = layer.bf16_to_f64(h_bits[m])
        # a bf16 tie may fall either way if the two silu evaluations differ in the last ulp
        for i in range(I):
            assert got_h[i] == hs[i] or abs(got_h[i] - hs[i]) <= 2 ** -7 * abs(hs[i]), i
        mismatch = sum(got_h[i] != hs[i] for i in range(I))
        assert mismatch <= 1
        if mismatch == 0:
            for r in range(H):
                ref = math.fsum(D[r][i] * hs[i] for i in range(I))
                assert abs(d[m, r] - ref) <= 1e-12 * max(1.0, abs(ref))


def _small_layer(seed=0, M=5, k=3, E=6, H=64, I=32):
    rng = np.random.default_rng(seed)
    experts = [_tiny_expert(1000 * seed + e, H, I) for e in range(E)]
    x = synthetic.bf16_from_f32(rng.standard_normal((M, H)).astype(np.float32))
    l = rng.standard_normal((M, E))
    ids, w, _, _ = layer.route(l, k)
    return x, ids, w, experts


def test_combine_hot_plus_cold_equals_full():
    x, ids, w, experts = _small_layer()
    rng = np.random.default_rng(5)
    for trial in range(4):
        e2s = np.where(rng.random(6) < 0.5, -1, rng.permutation(6))
        out = layer.layer_forward(x, ids, w, experts, e2s)
        assert np.allclose(out["y_hot"] + out["y_cold"], out["y_full"], rtol=1e-12, atol=1e-15)
        cold = [m * ids.shape[1] + j for m in range(ids.shape[0]) for j in range(ids.shape[1])
                if e2s[ids[m, j]] < 0]
        assert list(out["cold_routes"]) == cold


def test_combine_all_hot_all_cold_and_relabel():
    x, ids, w, experts = _small_layer(seed=2)
    full = layer.layer_forward(x, ids, w, experts, None)
    hot = layer.layer_forward(x, ids, w, experts, np.arange(6))
    assert np.array_equal(full["y_hot"], full["y_full"]) and not full["y_cold"].any()
    assert np.array_equal(hot["y_hot"], full["y_full"]) and hot["cold_routes"].size == 0
    cold = layer.layer_forward(x, ids, w, experts, np.full(6, -1))
    assert not cold["y_hot"].any()
    assert cold["cold_routes"].size == ids.size
    relabel = layer.layer_forward(x, ids, w, experts, np.array([5, 3, 1, 0, 2, 4]))
    assert np.array_equal(relabel["y_hot"], full["y_full"])


def test_combine_is_weighted_sum_of_expert_outputs():
    x, ids, w, experts = _small_layer(seed=3, M=2, k=2)
    out = layer.layer_forward(x, ids, w, experts, None)
    xf = layer.bf16_to_f64(x)
    for m in range(2):
        terms = []
        for j in range(2):
            _, d = layer.expert_ffn(xf[m:m + 1], layer.dequantize_expert(experts[ids[m, j]]))
            terms.append(w[m, j] * d[0])
        assert np.allclose(out["y_full"][m], terms[0] + terms[1], rtol=1e-13, atol=1e-15)


def test_buckets_invariants_and_stability():
    rng = np.random.default_rng(7)
    for M, k, E in ((1, 4, 32), (8, 10, 512), (64, 10, 512), (3, 2, 3)):
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(M)])
        counts, offsets, perm = layer.buckets(ids, E)
        flat = ids.reshape(-1)
        assert counts.sum() == M * k and offsets[-1] == M * k and offsets[0] == 0
        assert np.all(np.diff(offsets) == counts)
        assert sorted(perm.tolist()) == list(range(M * k))
        for e in range(E):
            members = perm[offsets[e]:offsets[e + 1]]
            assert np.all(flat[members] == e)
            assert np.all(np.diff(members) > 0)
        assert np.array_equal(counts, np.bincount(flat, minlength=E))
