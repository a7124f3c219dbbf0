"""GPU parity of the generic expert path (bf16, block FP8, NVFP4 experts) against the oracle.

The same slot cache, route table and combine as MXFP4, with the formats' own decode; the bars
are those of the MXFP4 tests: outputs within rel-L2 1e-3 and max-abs 2e-2 * max|ref|, cold
reports exact, repeated calls bit-identical.
"""
import numpy as np
import pytest
import torch

import synthetic
from expert_offloaded_routed_amd import binding as B
from expert_offloaded_routed_amd import layer as L
from oracle import layer as O

from gpu_common import close_enough, compare_routes, no_device_errors, say

pytestmark = pytest.mark.gpu

FORMATS = ["bf16", "fp8_block", "nvfp4"]

# Ragged shape: H = 320 (5 chunks of 64), I = 160 (FP8 scale blocks of 128 + 32 along both
# dimensions, NVFP4 rows of 10 scales), 16 experts, top-4.
RAGGED = synthetic.Workload("formats_ragged", 6, 320, 160, 16, 4, (1, 5, 70), 16)
GPTOSS = synthetic.WORKLOADS["gptoss20b_decode"]


def _dev(a):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _experts(wl, fmt, which):
    return dict(zip(which, synthetic.experts_canonical(wl, 0, which, fmt=fmt)))


def _call(shape, x, ids, w, e2s, slots, buf, M):
    B.moe_experts_forward(shape, _dev(x), M, _dev(np.ascontiguousarray(ids, np.int32)),
                          _dev(np.ascontiguousarray(w, np.float32)),
                          None if e2s is None else _dev(np.ascontiguousarray(e2s, np.int32)),
                          slots, buf.y, buf.cold_count, buf.cold_routes, buf.ws)
    torch.cuda.synchronize()
    no_device_errors(buf.ws)
    cc = int(buf.cold_count.item())
    return buf.y[:M].cpu().numpy(), cc, buf.cold_routes[:cc].cpu().numpy()


@pytest.mark.parametrize("fmt", FORMATS)
def test_format_ragged_shape_cold_maps_and_layer(fmt):
    wl = RAGGED
    experts = _experts(wl, fmt, range(wl.n_experts))
    shape = B.make_shape(wl.hidden, wl.inter, wl.n_experts, wl.top_k, wl.n_experts, fmt)
    assert B.moe_layer_launches(shape, 1) == 4
    bank = L.pack_bank(shape, [experts[e] for e in range(wl.n_experts)])
    rng = np.random.default_rng(21)
    slot_expert = rng.permutation(wl.n_experts).astype(np.int32)
    slots = L.device_slots(bank, slot_expert)
    wr = synthetic.router_weights(wl)
    buf = L.Buffers(shape, 70)
    for M in (1, 5, 70):
        say(f"{fmt} ragged M={M}")
        x = synthetic.activations(wl, M, M)
        ids_ref, w_ref, _, _ = O.route(O.router_logits(x, wr), wl.top_k)
        e2s = np.empty(wl.n_experts, np.int32)
        e2s[slot_expert] = np.arange(wl.n_experts)
        y, cc, _ = _call(shape, x, ids_ref, w_ref, e2s, slots, buf, M)
        ref = O.layer_forward(x, ids_ref, w_ref, experts)
        close_enough(y, ref["y_full"], f"{fmt} M={M} all hot")
        assert cc == 0
        y2, _, _ = _call(shape, x, ids_ref, w_ref, e2s, slots, buf, M)
        assert np.array_equal(y, y2)
        # a third of the experts cold
        e2s[rng.random(wl.n_experts) < 0.35] = -1
        y, cc, cold = _call(shape, x, ids_ref, w_ref, e2s, slots, buf, M)
        ref = O.layer_forward(x, ids_ref, w_ref, experts, e2s)
        assert cc == len(ref["cold_routes"]) and np.array_equal(cold, ref["cold_routes"])
        if np.linalg.norm(ref["y_hot"]) > 0:
            close_enough(y, ref["y_hot"], f"{fmt} M={M} part cold")
    say(f"{fmt} ragged: whole layer with the router and the residual")
    M = 5
    x = synthetic.activations(wl, M, 99)
    e2s = np.empty(wl.n_experts, np.int32)
    e2s[slot_expert] = np.arange(wl.n_experts)
    xd = _dev(x)
    x_next = torch.zeros_like(xd)
    B.moe_layer_forward_residual(shape, xd, M, _dev(wr), None, _dev(e2s), slots, buf.ids, buf.w,
                                 buf.y, buf.cold_count, buf.cold_routes, x_next, buf.ws)
    torch.cuda.synchronize()
    no_device_errors(buf.ws)
    ids = buf.ids[:M].cpu().numpy()
    w = buf.w[:M].cpu().numpy()
    _, ids_ref, w_ref = compare_routes(ids, w, O.router_logits(x, wr), wl.top_k)
    y = buf.y[:M].cpu().numpy()
    close_enough(y, O.layer_forward(x, ids_ref, w_ref, experts)["y_full"], f"{fmt} layer")
    # the residual equals the library's separate residual kernel on the same y, bitwise
    nxt_ref = torch.zeros_like(xd)
    B.moe_residual_bf16(xd, buf.y, nxt_ref, M * wl.hidden)
    torch.cuda.synchronize()
    assert torch.equal(x_next, nxt_ref)


@pytest.mark.parametrize("fmt", FORMATS)
def test_format_edge_cases(fmt):
    wl = RAGGED
    experts = _experts(wl, fmt, range(wl.n_experts))
    shape = B.make_shape(wl.hidden, wl.inter, wl.n_experts, wl.top_k, wl.n_experts, fmt)
    slots = L.device_slots(L.pack_bank(shape, [experts[e] for e in range(wl.n_experts)]))
    buf = L.Buffers(shape, 8)
    say(f"{fmt} edge: M = 0")
    buf.cold_count.fill_(77)
    B.moe_experts_forward(shape, None, 0, None, None, None, slots, None, buf.cold_count, None, buf.ws)
    torch.cuda.synchronize()
    assert int(buf.cold_count.item()) == 0
    say(f"{fmt} edge: all cold")
    M = 3
    x = synthetic.activations(wl, M, 7)
    rng = np.random.default_rng(2)
    ids = np.stack([rng.choice(wl.n_experts, wl.top_k, replace=False) for _ in range(M)])
    w = rng.random((M, wl.top_k)).astype(np.float32)
    buf.y.fill_(5.0)
    y, cc, cold = _call(shape, x, ids, w, np.full(wl.n_experts, -1, np.int32), slots, buf, M)
    assert cc == M * wl.top_k and np.array_equal(cold, np.arange(M * wl.top_k))
    assert not y.any()
    say(f"{fmt} edge: one expert takes every route of 8 tokens (k = 1)")
    shp1 = B.make_shape(wl.hidden, wl.inter, wl.n_experts, 1, wl.n_experts, fmt)
    b1 = L.Buffers(shp1, 8)
    x = synthetic.activations(wl, 8, 8)
    ids = np.full((8, 1), 5, np.int32)
    w = np.ones((8, 1), np.float32)
    y, _, _ = _call(shp1, x, ids, w, None, slots, b1, 8)
    close_enough(y, O.layer_forward(x, ids, w, experts)["y_full"], f"{fmt} k=1 one expert")


@pytest.mark.parametrize("fmt", FORMATS)
def test_format_gptoss_shape_full_size(fmt):
    """GPT-OSS-20B's layer shape (H = I = 2880) with four experts of the format in four slots
    and the other 28 cold: the launch configuration of the format's decode line."""
    wl = GPTOSS
    routed = [3, 11, 17, 30]
    experts = _experts(wl, fmt, routed)
    shape = B.make_shape(wl.hidden, wl.inter, wl.n_experts, wl.top_k, 4, fmt)
    slot_expert = np.array(routed, np.int32)
    bank = L.pack_bank(shape, [experts[e] for e in routed])
    slots = L.device_slots(bank)
    e2s = np.full(wl.n_experts, -1, np.int32)
    e2s[slot_expert] = np.arange(4)
    buf = L.Buffers(shape, 8)
    rng = np.random.default_rng(8)
    for M in (1, 8):
        say(f"{fmt} gptoss shape M={M}")
        x = synthetic.activations(wl, M, 5 + M)
        ids = np.stack([rng.permutation(routed)[:wl.top_k] for _ in range(M)]).astype(np.int32)
        w = rng.random((M, wl.top_k)).astype(np.float32)
        w /= w.sum(axis=1, keepdims=True)
        y, cc, _ = _call(shape, x, ids, w, e2s, slots, buf, M)
        assert cc == 0
        close_enough(y, O.layer_forward(x, ids, w, experts)["y_full"], f"{fmt} gptoss M={M}")
