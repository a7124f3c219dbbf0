"""Pins of the oracle's router, softmax/top-k/renormalise and bf16 helpers.

Brute force over every k-subset on the tiny layer (E=8, k=2), closed forms of the renormalised
weights, pure-Python dot products, torch's float->bfloat16 rounding as a library check.
"""
import itertools
import math

import numpy as np
import torch

import synthetic
from oracle import layer


def _tiny_logits(seed=0, M=64):
    wl = synthetic.WORKLOADS["tiny"]
    x = synthetic.activations(wl, M, seed)
    wr = synthetic.router_weights(wl)
    return x, wr, layer.router_logits(x, wr)


def test_router_logits_match_python_loops():
    wl = synthetic.WORKLOADS["tiny"]
    x = synthetic.activations(wl, 3, 7)
    wr = synthetic.router_weights(wl)
    bias = np.linspace(-1, 1, wl.n_experts).astype(np.float32)
    l = layer.router_logits(x, wr, bias)
    xf = layer.bf16_to_f64(x)
    wf = layer.bf16_to_f64(wr)
    for m in range(3):
        for e in range(wl.n_experts):
            ref = math.fsum(float(xf[m, h]) * float(wf[e, h]) for h in range(wl.hidden))
            ref += float(np.float32(bias[e]))
            assert abs(l[m, e] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_topk_brute_force_subsets():
    _, _, l = _tiny_logits()
    k = 2
    ids, w, gap, _ = layer.route(l, k)
    E = l.shape[1]
    for m in range(l.shape[0]):
        p = [math.exp(v - max(l[m])) for v in l[m]]
        z = math.fsum(p)
        p = [v / z for v in p]
        winners = [S for S in itertools.combinations(range(E), k)
                   if min(p[i] for i in S) > max(p[i] for i in range(E) if i not in S)]
        assert len(winners) == 1
        assert set(ids[m]) == set(winners[0])
        assert p[ids[m][0]] >= p[ids[m][1]]
        # closed form: renormalised weights are the softmax of the kept logits
        kept = [l[m, i] for i in ids[m]]
        den = math.fsum(math.exp(v - kept[0]) for v in kept)
        for j in range(k):
            assert abs(w[m, j] - math.exp(kept[j] - kept[0]) / den) < 1e-13
        assert abs(w[m].sum() - 1.0) < 1e-12
        assert gap[m] > 0


def test_topk_ties_go_to_lower_id_and_k_equals_E():
    l = np.array([[0.0, 3.0, 3.0, 1.0, 3.0, -1.0]])
    ids, w, gap, inner = layer.route(l, 2)
    assert list(ids[0]) == [1, 2]
    assert gap[0] == 0.0 and inner[0, 0] == 0.0
    assert np.allclose(w[0], [0.5, 0.5], atol=0, rtol=1e-15)
    ids, w, gap, _ = layer.route(l, 6)
    assert list(ids[0]) == [1, 2, 4, 3, 0, 5]
    assert gap[0] == np.inf


def test_softmax_first_equals_topk_first():
    _, _, l = _tiny_logits(seed=3, M=32)
    ids, w, _, _ = layer.route(l, 3)
    for m in range(l.shape[0]):
        top = np.argsort(-l[m], kind="stable")[:3]
        z = np.exp(l[m, top] - l[m, top].max())
        assert list(top) == list(ids[m])
        assert np.allclose(z / z.sum(), w[m], rtol=1e-14, atol=0)


def test_bf16_to_f64_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0x0001, 0x8000, 0x3FC0], dtype=np.uint16)
    got = layer.bf16_to_f64(bits)
    assert list(got[:3]) == [1.0, -2.0, math.inf]
    assert got[3] == 2.0 ** -133
    assert got[4] == 0.0 and math.copysign(1, got[4]) == -1
    assert got[5] == 1.5


def test_f64_to_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    a = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-39,
                        rng.standard_normal(2000) * 1e38]).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = layer.f64_to_bf16_rne(a.astype(np.float64))
    assert np.array_equal(got, ref)


def test_f64_to_bf16_halfway_cases():
    one = 1.0
    q = 2.0 ** -7  # bf16 spacing at 1.0
    cases = {
        one + q / 2: 0x3F80,            # tie -> even (1.0)
        one + 3 * q / 2: 0x3F82,        # tie -> even (1 + 2q)
        one + q / 2 + 2.0 ** -40: 0x3F81,  # just above the tie: up (not representable in fp32)
        -(one + q / 2): 0xBF80,
        2.0 ** -134: 0x0000,            # half of the smallest subnormal: tie to even zero
        3 * 2.0 ** -134: 0x0002,        # 1.5 subnormal steps: tie to even (2 steps)
        3.5e38: 0x7F80,                 # overflow -> inf
    }
    for v, bits in cases.items():
        assert int(layer.f64_to_bf16_rne(np.array([v]))[0]) == bits, v
