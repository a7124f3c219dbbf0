"""GPU parity of libmoe against the CPU oracle, through the C ABI (needs an MI355X).

Bars: top-k ids bit-exact (near-ties counted and excluded), weights and outputs within
rel-L2 1e-3 and max-abs 2e-2 * max|ref|, bucket counts/offsets, cold reports and slot
bookkeeping bit-exact.
"""
import numpy as np
import pytest
import torch

import synthetic
from expert_offloaded_routed_amd import binding as B
from expert_offloaded_routed_amd import layer as L
from oracle import layer as O
from oracle.cache_policy import LRU, SlotCachePolicy

from gpu_common import (close_enough, compare_routes, device_errors, no_device_errors,
                        oracle_weights_for, paths_agree, popularity_placement, routed_counts, say)

pytestmark = pytest.mark.gpu


def _shape(wl, n_slots=None):
    return B.make_shape(wl.hidden, wl.inter, wl.n_experts, wl.top_k, n_slots or wl.n_slots)


def _dev(a):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class Layer:
    """One layer's experts (canonical, host) and all-resident device slots."""

    def __init__(self, wl, layer=0):
        self.wl = wl
        self.layer = layer
        self.experts = synthetic.experts_canonical(wl, layer, range(wl.n_experts))
        self.shape = _shape(wl, max(wl.n_slots, wl.n_experts))
        self.bank = L.pack_bank(self.shape, self.experts)
        self.slots = L.device_slots(self.bank)
        self.wr = synthetic.router_weights(wl, layer)

    def slots_for(self, slot_expert):
        """A slot array holding bank[slot_expert[s]] in slot s."""
        return L.device_slots(self.bank, slot_expert, len(slot_expert))


@pytest.fixture(scope="module")
def tiny():
    return Layer(synthetic.WORKLOADS["tiny"])


@pytest.fixture(scope="module")
def gptoss():
    return Layer(synthetic.WORKLOADS["gptoss20b_decode"])


@pytest.fixture(scope="module")
def e512():
    return Layer(synthetic.WORKLOADS["e512_verify_stack"])


def run_route(shape, x, wr, bias, M, buf):
    B.moe_route(shape, _dev(x), M, _dev(wr), None if bias is None else _dev(bias), buf.ids, buf.w, buf.ws)
    torch.cuda.synchronize()
    no_device_errors(buf.ws)
    return buf.ids[:M].cpu().numpy(), buf.w[:M].cpu().numpy()


def run_experts(shape, x, ids, w, e2s, slots, buf, M):
    B.moe_experts_forward(shape, _dev(x), M, _dev(np.ascontiguousarray(ids, np.int32)),
                          _dev(np.ascontiguousarray(w, np.float32)),
                          None if e2s is None else _dev(np.ascontiguousarray(e2s, np.int32)),
                          slots, buf.y, buf.cold_count, buf.cold_routes, buf.ws)
    torch.cuda.synchronize()
    no_device_errors(buf.ws)
    cc = int(buf.cold_count.item())
    return buf.y[:M].cpu().numpy(), cc, buf.cold_routes[:cc].cpu().numpy()


# ---------------------------------------------------------------------------------------------
def test_tiny_route_buckets_and_layer(tiny):
    wl = tiny.wl
    M = wl.tokens[0]
    say("tiny: route + buckets + layer, M =", M)
    buf = L.Buffers(tiny.shape, M)
    x = synthetic.activations(wl, M, 0)
    ids, w = run_route(tiny.shape, x, tiny.wr, None, M, buf)
    excluded, ids_ref, w_ref = compare_routes(ids, w, O.router_logits(x, tiny.wr), wl.top_k)
    assert excluded == 0
    # buckets
    counts = torch.zeros(wl.n_experts, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(wl.n_experts + 1, dtype=torch.int32, device="cuda")
    perm = torch.zeros(M * wl.top_k, dtype=torch.int32, device="cuda")
    B.moe_bucket_routes(tiny.shape, _dev(ids_ref.astype(np.int32)), M, None, counts, offsets, perm,
                        buf.cold_count, buf.cold_routes, buf.ws)
    torch.cuda.synchronize()
    no_device_errors(buf.ws)
    c_ref, o_ref, p_ref = O.buckets(ids_ref, wl.n_experts)
    assert np.array_equal(counts.cpu().numpy(), c_ref)
    assert np.array_equal(offsets.cpu().numpy(), o_ref)
    pg = perm.cpu().numpy()
    for e in range(wl.n_experts):
        assert sorted(pg[o_ref[e]:o_ref[e + 1]]) == sorted(p_ref[o_ref[e]:o_ref[e + 1]])
    assert int(buf.cold_count.item()) == 0
    # expert FFNs + combine on the oracle's routes
    y, cc, _ = run_experts(tiny.shape, x, ids_ref, w_ref, None, tiny.slots, buf, M)
    ref = O.layer_forward(x, ids_ref, w_ref, tiny.experts)
    close_enough(y, ref["y_full"], "tiny y")
    assert cc == 0


@pytest.mark.parametrize("extra", [0, 1, 37])
def test_bucket_routes_many_routes(tiny, extra):
    """Bucketing of more routes than its one workgroup keeps in registers (8 per thread): the
    counts, offsets, per-expert route sets and the ascending cold list against their
    definitions, with every other expert cold and a skewed expert choice."""
    wl = tiny.wl
    E, k = wl.n_experts, wl.top_k
    M = 8 * 1024 // k + extra
    say("bucket routes: M =", M, "routes =", M * k)
    rng = np.random.default_rng(4100 + extra)
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(M)]).astype(np.int32)
    e2s = np.arange(E, dtype=np.int32)
    e2s[1::2] = -1
    buf = L.Buffers(tiny.shape, M)
    counts = torch.zeros(E, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.zeros(M * k, dtype=torch.int32, device="cuda")
    B.moe_bucket_routes(tiny.shape, _dev(ids), M, _dev(e2s), counts, offsets, perm, buf.cold_count,
                        buf.cold_routes, buf.ws)
    torch.cuda.synchronize()
    no_device_errors(buf.ws)
    c_ref, o_ref, p_ref = O.buckets(ids, E)
    assert np.array_equal(counts.cpu().numpy(), c_ref)
    assert np.array_equal(offsets.cpu().numpy(), o_ref)
    pg = perm.cpu().numpy()
    for e in range(E):
        assert np.array_equal(np.sort(pg[o_ref[e]:o_ref[e + 1]]), np.sort(p_ref[o_ref[e]:o_ref[e + 1]]))
    cold_ref = np.flatnonzero(e2s[ids.reshape(-1)] < 0)
    cc = int(buf.cold_count.item())
    assert cc == len(cold_ref)
    assert np.array_equal(buf.cold_routes[:cc].cpu().numpy(), cold_ref)


def test_tiny_cold_maps_and_slot_relabelling(tiny):
    wl = tiny.wl
    rng = np.random.default_rng(4)
    M = 7
    x = synthetic.activations(wl, M, 3)
    ids_ref, w_ref, _, _ = O.route(O.router_logits(x, tiny.wr), wl.top_k)
    shape = _shape(wl, 8)
    buf = L.Buffers(shape, M)
    base = None
    for trial in range(5):
        say("tiny cold map trial", trial)
        slot_expert = rng.permutation(wl.n_experts).astype(np.int32)
        e2s = np.empty(wl.n_experts, np.int32)
        e2s[slot_expert] = np.arange(wl.n_experts)
        if trial > 0:
            e2s[rng.random(wl.n_experts) < 0.4] = -1
        slots = tiny.slots_for(slot_expert)
        y, cc, cold = run_experts(shape, x, ids_ref, w_ref, e2s, slots, buf, M)
        ref = O.layer_forward(x, ids_ref, w_ref, tiny.experts, e2s)
        assert cc == len(ref["cold_routes"]) and np.array_equal(cold, ref["cold_routes"])
        if np.linalg.norm(ref["y_hot"]) > 0:
            close_enough(y, ref["y_hot"], f"tiny y_hot trial {trial}")
        if trial == 0:
            base = y.copy()
            close_enough(y, ref["y_full"], "tiny relabelled")
    # a second relabelling with every expert hot gives bit-identical output
    slot_expert = np.roll(np.arange(wl.n_experts), 3).astype(np.int32)
    e2s = np.empty(wl.n_experts, np.int32)
    e2s[slot_expert] = np.arange(wl.n_experts)
    y, _, _ = run_experts(shape, x, ids_ref, w_ref, e2s, tiny.slots_for(slot_expert), buf, M)
    assert np.array_equal(y, base)


def test_tiny_edge_cases(tiny):
    wl = tiny.wl
    shape = tiny.shape
    buf = L.Buffers(shape, 8)
    say("edge: M = 0")
    B.moe_route(shape, _dev(synthetic.activations(wl, 1, 0)), 0, _dev(tiny.wr), None, buf.ids, buf.w, buf.ws)
    buf.cold_count.fill_(77)
    B.moe_experts_forward(shape, None, 0, None, None, None, tiny.slots, None, buf.cold_count, None, buf.ws)
    torch.cuda.synchronize()
    assert int(buf.cold_count.item()) == 0
    say("edge: all cold")
    M = 3
    x = synthetic.activations(wl, M, 11)
    ids_ref, w_ref, _, _ = O.route(O.router_logits(x, tiny.wr), wl.top_k)
    buf.y.fill_(5.0)
    y, cc, cold = run_experts(shape, x, ids_ref, w_ref, np.full(wl.n_experts, -1, np.int32), tiny.slots, buf, M)
    assert cc == M * wl.top_k and np.array_equal(cold, np.arange(M * wl.top_k))
    assert not y.any()
    say("edge: ragged M and repeated calls")
    for M in (1, 2, 3, 5, 8):
        x = synthetic.activations(wl, M, 20 + M)
        ids, w = run_route(shape, x, tiny.wr, None, M, buf)
        ex, ids_ref, w_ref = compare_routes(ids, w, O.router_logits(x, tiny.wr), wl.top_k)
        y1, _, _ = run_experts(shape, x, ids_ref, w_ref, None, tiny.slots, buf, M)
        y2, _, _ = run_experts(shape, x, ids_ref, w_ref, None, tiny.slots, buf, M)
        assert np.array_equal(y1, y2)
        close_enough(y1, O.layer_forward(x, ids_ref, w_ref, tiny.experts)["y_full"], f"tiny M={M}")
    say("edge: k = E (every expert routed)")
    shp = B.make_shape(wl.hidden, wl.inter, wl.n_experts, wl.n_experts, wl.n_experts)
    b2 = L.Buffers(shp, 2)
    x = synthetic.activations(wl, 2, 40)
    ids, w = run_route(shp, x, tiny.wr, None, 2, b2)
    _, ids_ref, w_ref = compare_routes(ids, w, O.router_logits(x, tiny.wr), wl.n_experts)
    y, _, _ = run_experts(shp, x, ids_ref, w_ref, None, tiny.slots, b2, 2)
    close_enough(y, O.layer_forward(x, ids_ref, w_ref, tiny.experts)["y_full"], "tiny k=E")


def test_gptoss20b_decode_full_size(gptoss):
    wl = gptoss.wl
    shape = gptoss.shape
    buf = L.Buffers(shape, 1)
    bias = synthetic.zipf_bias(wl)
    steps = wl.steps
    xs = np.concatenate([synthetic.activations(wl, 1, t) for t in range(steps)])
    say("gptoss20b: routing 256 M=1 decode steps")
    ids = np.zeros((steps, wl.top_k), np.int32)
    w = np.zeros((steps, wl.top_k), np.float32)
    for t in range(steps):
        ids[t], w[t] = run_route(shape, xs[t:t + 1], gptoss.wr, bias, 1, buf)
    excluded, ids_ref, w_ref = compare_routes(ids, w, O.router_logits(xs, gptoss.wr, bias), wl.top_k)
    say("gptoss20b: near-tie tokens excluded:", excluded)
    assert excluded <= 2
    for t in (0, 1, 97, 255):
        say("gptoss20b: expert FFNs, step", t)
        y, cc, _ = run_experts(shape, xs[t:t + 1], ids_ref[t:t + 1], w_ref[t:t + 1], None, gptoss.slots, buf, 1)
        ref = O.layer_forward(xs[t:t + 1], ids_ref[t:t + 1], w_ref[t:t + 1], gptoss.experts)
        close_enough(y, ref["y_full"], f"gptoss20b step {t}")
        assert cc == 0


@pytest.mark.parametrize("M", [1, 4, 8])
def test_e512_verify_half_resident(e512, M):
    wl = e512.wl
    say("e512: placement from warm-up routing, M =", M)
    counts = routed_counts(wl, 0, 256)
    slot_expert = popularity_placement(counts, wl.n_slots)
    e2s = np.full(wl.n_experts, -1, np.int32)
    e2s[slot_expert] = np.arange(wl.n_slots)
    shape = _shape(wl, wl.n_slots)
    # one token: router + fused kernel; 4 and 8 tokens: router, top-k / bucketing, gate/up, down
    # + combine (the down GEMV shares each row tile's experts between two workgroups, which hand
    # rows over through the workspace)
    assert B.moe_layer_launches(shape, M) == {1: 2, 4: 4, 8: 4}[M]
    slots = e512.slots_for(slot_expert)
    buf = L.Buffers(shape, M)
    bias = synthetic.zipf_bias(wl)
    x = synthetic.activations(wl, M, 5)
    ids, w = run_route(shape, x, e512.wr, bias, M, buf)
    excluded, ids_ref, w_ref = compare_routes(ids, w, O.router_logits(x, e512.wr, bias), wl.top_k)
    assert excluded == 0
    y, cc, cold = run_experts(shape, x, ids_ref, w_ref, e2s, slots, buf, M)
    ref = O.layer_forward(x, ids_ref, w_ref, e512.experts, e2s)
    assert cc == len(ref["cold_routes"]) and np.array_equal(cold, ref["cold_routes"])
    close_enough(y, ref["y_hot"], f"e512 M={M} y_hot")
    # the whole layer call (for one token: router + the fused kernel over the 10 routes)
    lb = L.Buffers(shape, M)
    B.moe_layer_forward(shape, _dev(x), M, _dev(e512.wr), _dev(bias), _dev(e2s), slots, lb.ids, lb.w,
                        lb.y, lb.cold_count, lb.cold_routes, lb.ws)
    torch.cuda.synchronize()
    no_device_errors(lb.ws)
    assert torch.equal(lb.ids[:M], buf.ids[:M]) and torch.equal(lb.w[:M], buf.w[:M])
    assert int(lb.cold_count.item()) == cc
    paths_agree(lb.y[:M].cpu().numpy(), y, f"e512 M={M} layer call")
    close_enough(lb.y[:M].cpu().numpy(), ref["y_hot"], f"e512 M={M} layer call y_hot")


def test_e512_prefill_sampled_tokens(e512):
    wl = synthetic.WORKLOADS["e512_prefill"]
    M = wl.tokens[0]
    shape = _shape(wl, wl.n_experts)
    buf = L.Buffers(shape, M)
    wr = synthetic.router_weights(wl)
    bias = synthetic.zipf_bias(wl)
    x = synthetic.activations(wl, M, 0)
    # the e512 fixture's experts belong to another workload: use this workload's own experts
    experts = synthetic.experts_canonical(wl, 0, range(wl.n_experts))
    slots = L.device_slots(L.pack_bank(shape, experts))
    say("e512 prefill: route M =", M)
    ids, w = run_route(shape, x, wr, bias, M, buf)
    excluded, ids_ref, w_ref = compare_routes(ids, w, O.router_logits(x, wr, bias), wl.top_k)
    say("e512 prefill: near-tie tokens excluded:", excluded)
    say("e512 prefill: experts")
    y, cc, _ = run_experts(shape, x, ids_ref, w_ref, None, slots, buf, M)
    assert cc == 0
    # every token of the call (the grouped GEMMs: 16 K chunks, Zipf-skewed experts that take
    # several 64-route passes, the split-h block-scaled down projection and the combine)
    ref = O.layer_forward(x, ids_ref, w_ref, experts)
    rel = close_enough(y, ref["y_full"], "e512 prefill, all 512 tokens")
    per_tok = np.linalg.norm(y - ref["y_full"], axis=1) / np.linalg.norm(ref["y_full"], axis=1)
    counts = np.bincount(ids_ref.reshape(-1), minlength=wl.n_experts)
    say(f"e512 prefill: rel-L2 over all {M} tokens {rel:.3e}, worst token {per_tok.max():.3e}; "
        f"busiest expert {counts.max()} routes ({-(-counts.max() // 64)} passes of 64)")
    # the whole layer call (router GEMM, top-k / bucketing, grouped gate/up, down, combine)
    lb = L.Buffers(shape, M)
    B.moe_layer_forward(shape, _dev(x), M, _dev(wr), _dev(bias), None, slots, lb.ids, lb.w, lb.y,
                        lb.cold_count, lb.cold_routes, lb.ws)
    torch.cuda.synchronize()
    no_device_errors(lb.ws)
    assert torch.equal(lb.ids[:M], buf.ids[:M]) and torch.equal(lb.w[:M], buf.w[:M])
    ids_l = lb.ids[:M].cpu().numpy()
    lg = O.router_logits(x, wr, bias)
    compare_routes(ids_l, lb.w[:M].cpu().numpy(), lg, wl.top_k)
    # the reference with the call's own top-k sets (equal to the oracle's except on near-ties)
    ref_l = O.layer_forward(x, ids_l, oracle_weights_for(lg, ids_l), experts)
    rel_l = close_enough(lb.y[:M].cpu().numpy(), ref_l["y_full"], "e512 prefill layer call")
    say(f"e512 prefill: layer call rel-L2 {rel_l:.3e}")


@pytest.mark.parametrize("M", [64, 130])
def test_tiny_grouped_gemm_every_token(tiny, M):
    """M >= 64 takes the grouped GEMM (MFMA) kernels: every token against the oracle, half the
    experts cold, 130 = two passes of 64 routes plus a ragged tail for the busiest experts; the
    layer entry point and the staged calls agree bitwise with the one-call path."""
    wl = tiny.wl
    say("tiny grouped GEMM: M =", M)
    shape = tiny.shape
    x = synthetic.activations(wl, M, 700 + M)
    ids_ref, w_ref, _, _ = O.route(O.router_logits(x, tiny.wr), wl.top_k)
    e2s = np.arange(wl.n_experts, dtype=np.int32)
    e2s[1::2] = -1
    buf = L.Buffers(shape, M)
    y, cc, cold = run_experts(shape, x, ids_ref, w_ref, e2s, tiny.slots, buf, M)
    ref = O.layer_forward(x, ids_ref, w_ref, tiny.experts, e2s)
    assert cc == len(ref["cold_routes"]) and np.array_equal(cold, ref["cold_routes"])
    close_enough(y, ref["y_hot"], f"tiny grouped M={M} y_hot")
    # all resident, through the layer entry point and the staged calls
    xd, wr = _dev(x), _dev(tiny.wr)
    a, c = L.Buffers(shape, M), L.Buffers(shape, M)
    B.moe_layer_forward(shape, xd, M, wr, None, None, tiny.slots, a.ids, a.w, a.y, a.cold_count,
                        a.cold_routes, a.ws)
    B.moe_route(shape, xd, M, wr, None, c.ids, c.w, c.ws)
    B.moe_experts_gateup(shape, xd, M, c.ids, c.w, None, tiny.slots, c.ws)
    B.moe_experts_down(shape, M, c.ids, c.w, None, tiny.slots, c.y, c.ws)
    torch.cuda.synchronize()
    no_device_errors(a.ws, c.ws)
    assert torch.equal(a.ids[:M], c.ids[:M]) and torch.equal(a.y[:M], c.y[:M])
    excluded, ids2, w2 = compare_routes(a.ids[:M].cpu().numpy(), a.w[:M].cpu().numpy(),
                                        O.router_logits(x, tiny.wr), wl.top_k)
    assert excluded == 0
    ref2 = O.layer_forward(x, ids2, w2, tiny.experts)
    close_enough(a.y[:M].cpu().numpy(), ref2["y_full"], f"tiny grouped layer M={M}")


def test_refill_copies_images_exactly(tiny):
    shape = tiny.shape
    say("refill: pinned bank -> slots")
    bank = L.pinned_bank(tiny.bank)
    slots = torch.zeros_like(tiny.slots)
    copy = torch.cuda.Stream()
    done = B.event_create()
    before = B.event_create()
    B.event_record(before)
    B.moe_slot_refill(shape, slots, bank, [3, 5, 0], [1, 7, 2], copy, before, done)
    B.stream_wait_event(torch.cuda.current_stream(), done)
    got = slots.cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(got[1], tiny.bank[3])
    assert np.array_equal(got[7], tiny.bank[5])
    assert np.array_equal(got[2], tiny.bank[0])
    assert not got[0].any()
    B.event_destroy(done)
    B.event_destroy(before)


def test_graph_capture_replays_match_eager(tiny):
    wl = tiny.wl
    shape = tiny.shape
    M = 4
    buf = L.Buffers(shape, M)
    x = _dev(synthetic.activations(wl, M, 0))
    wr = _dev(tiny.wr)
    say("graph: eager reference")
    B.moe_route(shape, x, M, wr, None, buf.ids, buf.w, buf.ws)
    B.moe_experts_forward(shape, x, M, buf.ids, buf.w, None, tiny.slots, buf.y, None, None, buf.ws)
    torch.cuda.synchronize()
    y_eager = buf.y[:M].clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    say("graph: capture")
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            B.moe_route(shape, x, M, wr, None, buf.ids, buf.w, buf.ws, stream=s)
            B.moe_experts_forward(shape, x, M, buf.ids, buf.w, None, tiny.slots, buf.y, None, None,
                                  buf.ws, stream=s)
    torch.cuda.synchronize()
    for rep in range(4):
        say("graph: replay", rep)
        buf.y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(buf.y[:M], y_eager)
        no_device_errors(buf.ws)
        # eager work between replays
        B.moe_experts_forward(shape, x, M, buf.ids, buf.w, None, tiny.slots, buf.y, None, None, buf.ws)
        torch.cuda.synchronize()


def test_slot_cache_pipeline_bookkeeping():
    """8-slot GPT-OSS-20B-shaped layer over 40 decode steps with LRU refills (lag 3): the
    published maps, refill plans and per-step cold counts equal the oracle's replay, and the
    hot-only outputs match on sampled steps."""
    wl = synthetic.WORKLOADS["gptoss20b_8slots"]
    steps, lag, D = 40, 3, 1
    shape = _shape(wl, wl.n_slots)
    say("cache pipeline: generating 32 experts")
    experts = synthetic.experts_canonical(wl, 0, range(wl.n_experts))
    bank_np = L.pack_bank(shape, experts)
    bank = L.pinned_bank(bank_np)
    ranks = synthetic.zipf_ranks(wl)
    init = np.argsort(ranks)[: wl.n_slots].astype(np.int32)  # ranks 1..8 in rank order
    slots = L.device_slots(bank_np, init, wl.n_slots)
    wr = synthetic.router_weights(wl)
    xs = [synthetic.activations(wl, 1, t) for t in range(steps)]
    biases = [synthetic.zipf_bias(wl, 0, synthetic.drift_shift(wl, t)) for t in range(steps)]
    # oracle replay
    ids_ref = [O.route(O.router_logits(xs[t], wr, biases[t]), wl.top_k)[0] for t in range(steps)]
    pol = SlotCachePolicy(wl.n_experts, wl.n_slots, init, policy=LRU, max_refills=2, lag=lag, max_pending=2)
    # GPU pipeline with the library's host policy
    cache = B.MoeCache(shape, lag_steps=lag, initial_slot_expert=init)
    buf = L.Buffers(shape, 1)
    copy = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    ids_host = []
    done_events = {}
    maps, plans, colds, ys = [], [], [], []
    wr_d = _dev(wr)
    for t in range(steps):
        obs = ids_host[t - D] if t - D >= 0 else None
        m_lib, plan, _ = cache.moe_cache_policy_step(t, obs)
        m_ref, plan_ref = pol.step(t, ids_ref[t - D] if t - D >= 0 else None)
        assert np.array_equal(m_lib, m_ref), t
        assert plan == plan_ref, t
        for ev in done_events.pop(t, []):  # refills visible now: compute waits for their copies
            B.stream_wait_event(comp, ev)
        e2s = _dev(m_lib)
        B.moe_route(shape, _dev(xs[t]), 1, wr_d, _dev(biases[t]), buf.ids, buf.w, buf.ws)
        B.moe_experts_forward(shape, _dev(xs[t]), 1, buf.ids, buf.w, e2s, slots, buf.y,
                              buf.cold_count, buf.cold_routes, buf.ws)
        after = B.event_create()
        B.event_record(after, comp)
        if plan:
            done = B.event_create()
            B.moe_slot_refill(shape, slots, bank, [p[0] for p in plan], [p[1] for p in plan], copy,
                              after, done)
            done_events.setdefault(plan[0][3], []).append(done)
        torch.cuda.synchronize()
        no_device_errors(buf.ws)
        ids_t = buf.ids[:1].cpu().numpy().copy()
        ids_host.append(ids_t)
        assert np.array_equal(ids_t, ids_ref[t]), t
        colds.append(int(buf.cold_count.item()))
        ys.append(buf.y[:1].cpu().numpy().copy())
        maps.append(m_lib)
        plans.append(plan)
    flat = [np.asarray(i).reshape(-1) for i in ids_ref]
    assert colds == [int((maps[t][flat[t]] < 0).sum()) for t in range(steps)]
    assert sum(len(p) for p in plans) > 0
    for t in (5, 20, 39):
        w_ref = O.route(O.router_logits(xs[t], wr, biases[t]), wl.top_k)[1]
        ref = O.layer_forward(xs[t], ids_ref[t], w_ref, experts, maps[t])
        if np.linalg.norm(ref["y_hot"]) > 0:
            close_enough(ys[t], ref["y_hot"], f"cache pipeline step {t}")
        else:
            assert not ys[t].any()
    cache.close()


def test_layer_forward_equals_route_plus_experts_and_stages(gptoss):
    """moe_layer_forward == moe_route + moe_experts_forward == bucket + gateup + down (bitwise,
    or, for one token, where the layer call is one fused launch, to rel-L2 1e-4), and all of
    them match the oracle; also with a cold expert map."""
    wl = gptoss.wl
    shape = gptoss.shape
    bias = synthetic.zipf_bias(wl)
    for M in (1, 3):
        say("layer_forward equivalence, M =", M)
        x = _dev(synthetic.activations(wl, M, 500 + M))
        wr = _dev(gptoss.wr)
        bd = _dev(bias)
        e2s_np = np.arange(wl.n_experts, dtype=np.int32)
        e2s_np[[1, 5, 9, 30]] = -1
        for e2s in (None, _dev(e2s_np)):
            a, b, c = L.Buffers(shape, M), L.Buffers(shape, M), L.Buffers(shape, M)
            B.moe_layer_forward(shape, x, M, wr, bd, e2s, gptoss.slots, a.ids, a.w, a.y, a.cold_count,
                                a.cold_routes, a.ws)
            B.moe_route(shape, x, M, wr, bd, b.ids, b.w, b.ws)
            B.moe_experts_forward(shape, x, M, b.ids, b.w, e2s, gptoss.slots, b.y, b.cold_count,
                                  b.cold_routes, b.ws)
            B.moe_route(shape, x, M, wr, bd, c.ids, c.w, c.ws)
            B.moe_bucket_routes(shape, c.ids, M, e2s, None, None, None, c.cold_count, c.cold_routes, c.ws)
            B.moe_experts_gateup(shape, x, M, c.ids, c.w, e2s, gptoss.slots, c.ws)
            B.moe_experts_down(shape, M, c.ids, c.w, e2s, gptoss.slots, c.y, c.ws)
            torch.cuda.synchronize()
            no_device_errors(a.ws, b.ws, c.ws)
            assert torch.equal(b.y[:M], c.y[:M])  # the same kernels, staged differently
            for other in (b, c):
                assert torch.equal(a.ids[:M], other.ids[:M]) and torch.equal(a.w[:M], other.w[:M])
                if B.moe_layer_launches(shape, M) <= 2:  # one token: the fused kernel
                    paths_agree(a.y[:M].cpu().numpy(), other.y[:M].cpu().numpy(), f"M={M}")
                else:
                    assert torch.equal(a.y[:M], other.y[:M])
                assert torch.equal(a.cold_count, other.cold_count)
            xn = synthetic.activations(wl, M, 500 + M)
            _, ids_ref, w_ref = compare_routes(a.ids[:M].cpu().numpy(), a.w[:M].cpu().numpy(),
                                               O.router_logits(xn, gptoss.wr, bias), wl.top_k)
            ref = O.layer_forward(xn, ids_ref, w_ref, gptoss.experts,
                                  None if e2s is None else e2s_np)
            close_enough(a.y[:M].cpu().numpy(), ref["y_hot"], f"layer_forward M={M}")
            assert int(a.cold_count.item()) == len(ref["cold_routes"])


def test_marked_layer_forward_and_residual(gptoss):
    """moe_layer_forward_marked gives the results of moe_layer_forward and ordered stage events;
    moe_residual_bf16 rounds x + y to bf16 exactly like float32 addition followed by RNE."""
    wl = gptoss.wl
    shape = gptoss.shape
    M = 2
    say("marked layer forward")
    x = _dev(synthetic.activations(wl, M, 900))
    wr, bd = _dev(gptoss.wr), _dev(synthetic.zipf_bias(wl))
    a, b = L.Buffers(shape, M), L.Buffers(shape, M)
    marks = [B.event_create(timing=True) for _ in range(4)]
    B.moe_layer_forward(shape, x, M, wr, bd, None, gptoss.slots, a.ids, a.w, a.y, None, None, a.ws)
    B.moe_layer_forward_marked(shape, x, M, wr, bd, None, gptoss.slots, b.ids, b.w, b.y, None, None,
                               b.ws, marks)
    torch.cuda.synchronize()
    no_device_errors(a.ws, b.ws)
    assert torch.equal(a.ids[:M], b.ids[:M]) and torch.equal(a.y[:M], b.y[:M])
    stages = [B.event_elapsed_ms(marks[j], marks[j + 1]) for j in range(3)]
    assert all(t >= 0 for t in stages), stages
    for e in marks:
        B.event_destroy(e)
    with pytest.raises(B.MoeError):
        B.moe_layer_forward_marked(shape, x, M, wr, bd, None, gptoss.slots, b.ids, b.w, b.y, None,
                                   None, b.ws, [0, 0, 0, 0])
    say("residual")
    n = 3 * 2880 + 1  # odd: the last thread handles one element
    rng = np.random.default_rng(3)
    xh = synthetic.bf16_from_f32(rng.standard_normal(n).astype(np.float32))
    yh = (rng.standard_normal(n) * 0.1).astype(np.float32)
    xd, yd = _dev(xh), torch.from_numpy(yh).cuda()
    out = torch.zeros(n, dtype=torch.int16, device="cuda")
    B.moe_residual_bf16(xd, yd, out, n)
    B.moe_residual_bf16(xd, yd, xd, n)  # in place
    torch.cuda.synchronize()
    xf = (xh.astype(np.uint32) << 16).view(np.float32)
    ref = synthetic.bf16_from_f32((xf + yh).astype(np.float32))
    assert np.array_equal(out.cpu().numpy().view(np.uint16), ref)
    assert np.array_equal(xd.cpu().numpy().view(np.uint16), ref)



def test_fused_decode_consecutive_tokens_and_maps(gptoss):
    """One-token layer calls run gate/up and down as one launch.  Over consecutive tokens
    (h of the previous token still in the workspace), with every expert hot, some top-k experts
    cold, all cold, and slots relabelled, the fused call agrees with moe_route +
    moe_experts_forward (to rel-L2 1e-4, bitwise on ids, weights and the cold report) and with
    the oracle to the parity bar."""
    wl = gptoss.wl
    shape = gptoss.shape
    assert B.moe_layer_launches(shape, 1) == 1  # the router runs inside the fused kernel
    bias = synthetic.zipf_bias(wl)
    wr, bd = _dev(gptoss.wr), _dev(bias)
    E = wl.n_experts
    rng = np.random.default_rng(11)
    perm = rng.permutation(E).astype(np.int32)  # expert e in slot perm[e]
    part = np.arange(E, dtype=np.int32)
    part[rng.choice(E, E // 2, replace=False)] = -1
    maps = [("identity", None, None), ("half cold", part, gptoss.slots),
            ("all cold", np.full(E, -1, np.int32), gptoss.slots),
            ("relabelled", perm, gptoss.slots_for(np.argsort(perm)))]
    a, b = L.Buffers(shape, 1), L.Buffers(shape, 1)
    for name, e2s_np, slots in maps:
        slots = gptoss.slots if slots is None else slots
        e2s = None if e2s_np is None else _dev(e2s_np)
        for t in range(6):
            say("fused decode:", name, "token", t)
            xn = synthetic.activations(wl, 1, 700 + t)
            x = _dev(xn)
            B.moe_layer_forward(shape, x, 1, wr, bd, e2s, slots, a.ids, a.w, a.y, a.cold_count,
                                a.cold_routes, a.ws)
            B.moe_route(shape, x, 1, wr, bd, b.ids, b.w, b.ws)
            B.moe_experts_forward(shape, x, 1, b.ids, b.w, e2s, slots, b.y, b.cold_count,
                                  b.cold_routes, b.ws)
            torch.cuda.synchronize()
            no_device_errors(a.ws, b.ws)
            assert torch.equal(a.ids[:1], b.ids[:1]) and torch.equal(a.w[:1], b.w[:1])
            paths_agree(a.y[:1].cpu().numpy(), b.y[:1].cpu().numpy(), name)
            cc = int(a.cold_count.item())
            assert cc == int(b.cold_count.item())
            assert torch.equal(a.cold_routes[:cc], b.cold_routes[:cc])
            if t % 3 == 0:
                _, ids_ref, w_ref = compare_routes(a.ids[:1].cpu().numpy(), a.w[:1].cpu().numpy(),
                                                   O.router_logits(xn, gptoss.wr, bias), wl.top_k)
                ref = O.layer_forward(xn, ids_ref, w_ref, gptoss.experts, e2s_np)
                if name == "all cold":
                    assert not a.y[:1].any() and cc == wl.top_k
                else:
                    close_enough(a.y[:1].cpu().numpy(), ref["y_hot"], f"fused decode {name} {t}")
                assert cc == len(ref["cold_routes"])


@pytest.mark.parametrize("E,k", [(65, 3), (100, 7), (300, 16)])
def test_fused_decode_many_experts_route_table(E, k):
    """The one-token route table for 64 < E <= 512 (every wave ranks its 64 keys, the k best of
    each wave are ranked among themselves): on H = 256, I = 512 layers with E = 65, 100, 300 and
    k = 3, 7, 16, with all experts resident and with every third expert cold, the layer call
    (router + fused kernel) publishes bitwise the ids and weights of moe_route, agrees with the
    two-call path and matches the oracle."""
    import dataclasses
    base = synthetic.WORKLOADS["tiny"]
    wl = dataclasses.replace(base, name=f"tiny_e{E}_k{k}", n_experts=E, top_k=k, n_slots=E)
    shape = _shape(wl, E)
    assert B.moe_layer_launches(shape, 1) == 2  # the fused kernel takes the call
    gen = synthetic.experts_canonical(wl, 0, range(8))
    experts = [gen[e % 8] for e in range(E)]
    slots = L.device_slots(L.pack_bank(shape, experts))
    wr_np = synthetic.router_weights(wl)
    wr = _dev(wr_np)
    part = np.arange(E, dtype=np.int32)
    part[::3] = -1
    a, b = L.Buffers(shape, 1), L.Buffers(shape, 1)
    for name, e2s_np in (("identity", None), ("every third expert cold", part)):
        e2s = None if e2s_np is None else _dev(e2s_np)
        for t in range(4):
            say("fused decode, many experts:", E, k, name, "token", t)
            xn = synthetic.activations(wl, 1, 700 + t)
            x = _dev(xn)
            B.moe_layer_forward(shape, x, 1, wr, None, e2s, slots, a.ids, a.w, a.y,
                                a.cold_count, a.cold_routes, a.ws)
            B.moe_route(shape, x, 1, wr, None, b.ids, b.w, b.ws)
            B.moe_experts_forward(shape, x, 1, b.ids, b.w, e2s, slots, b.y, b.cold_count,
                                  b.cold_routes, b.ws)
            torch.cuda.synchronize()
            no_device_errors(a.ws, b.ws)
            assert torch.equal(a.ids[:1], b.ids[:1]) and torch.equal(a.w[:1], b.w[:1])
            assert int(a.cold_count.item()) == int(b.cold_count.item())
            paths_agree(a.y[:1].cpu().numpy(), b.y[:1].cpu().numpy(), f"E={E} k={k} {name}")
            _, ids_ref, w_ref = compare_routes(a.ids[:1].cpu().numpy(), a.w[:1].cpu().numpy(),
                                               O.router_logits(xn, wr_np), k)
            ref = O.layer_forward(xn, ids_ref, w_ref, experts, e2s_np)
            assert int(a.cold_count.item()) == len(ref["cold_routes"])
            close_enough(a.y[:1].cpu().numpy(), ref["y_hot"], f"fused E={E} k={k} {name} {t}")


def test_fused_decode_two_down_units_more_routes():
    """The fused one-token kernel with the router inside where a workgroup holds two down units
    and the token has more than four routes (H = 3072, I = 1024, E = 8, k = 6): y is then formed
    from the waves' sums in LDS rather than one wave per row.  Against the oracle and the
    two-call path, all experts resident and with every third expert cold."""
    import dataclasses
    k = 6
    wl = dataclasses.replace(synthetic.WORKLOADS["tiny"], name="wide_k6", hidden=3072, inter=1024,
                             n_experts=8, top_k=k, n_slots=8)
    shape = _shape(wl, wl.n_experts)
    assert B.moe_layer_launches(shape, 1) == 1  # the router runs inside the fused kernel
    say("fused decode, H = 3072, k = 6: generating 8 experts")
    experts = synthetic.experts_canonical(wl, 0, range(wl.n_experts))
    slots = L.device_slots(L.pack_bank(shape, experts))
    wr_np = synthetic.router_weights(wl)
    wr = _dev(wr_np)
    part = np.arange(wl.n_experts, dtype=np.int32)
    part[::3] = -1
    a, b = L.Buffers(shape, 1), L.Buffers(shape, 1)
    for name, e2s_np in (("identity", None), ("every third expert cold", part)):
        e2s = None if e2s_np is None else _dev(e2s_np)
        for t in range(3):
            say("fused decode, H = 3072, k = 6:", name, "token", t)
            xn = synthetic.activations(wl, 1, 900 + t)
            x = _dev(xn)
            B.moe_layer_forward(shape, x, 1, wr, None, e2s, slots, a.ids, a.w, a.y,
                                a.cold_count, a.cold_routes, a.ws)
            B.moe_route(shape, x, 1, wr, None, b.ids, b.w, b.ws)
            B.moe_experts_forward(shape, x, 1, b.ids, b.w, e2s, slots, b.y, b.cold_count,
                                  b.cold_routes, b.ws)
            torch.cuda.synchronize()
            no_device_errors(a.ws, b.ws)
            assert torch.equal(a.ids[:1], b.ids[:1]) and torch.equal(a.w[:1], b.w[:1])
            assert int(a.cold_count.item()) == int(b.cold_count.item())
            paths_agree(a.y[:1].cpu().numpy(), b.y[:1].cpu().numpy(), f"H=3072 k=6 {name}")
            _, ids_ref, w_ref = compare_routes(a.ids[:1].cpu().numpy(), a.w[:1].cpu().numpy(),
                                               O.router_logits(xn, wr_np), k)
            ref = O.layer_forward(xn, ids_ref, w_ref, experts, e2s_np)
            assert int(a.cold_count.item()) == len(ref["cold_routes"])
            close_enough(a.y[:1].cpu().numpy(), ref["y_hot"], f"fused H=3072 k=6 {name} {t}")


def test_fused_decode_small_shape_and_graph_replays(tiny, gptoss):
    """The fused one-token kernel on a second shape (H = 256, I = 512, E = 8, k = 2: one unit of
    each kind per workgroup) against the oracle and the two-call path, over tokens whose top-k
    experts are all hot, partly cold or all cold; then one-token layer calls of both shapes
    captured in a HIP graph and replayed, with eager calls between the replays (the h rows are
    re-marked by the router of every call), each replay equal to the eager result."""
    wl, shape = tiny.wl, tiny.shape
    assert B.moe_layer_launches(shape, 1) == 1  # the router runs inside the fused kernel
    wr = _dev(tiny.wr)
    E = wl.n_experts
    part = np.arange(E, dtype=np.int32)
    part[1::2] = -1
    a, b = L.Buffers(shape, 1), L.Buffers(shape, 1)
    for name, e2s_np in (("identity", None), ("odd experts cold", part),
                         ("all cold", np.full(E, -1, np.int32))):
        e2s = None if e2s_np is None else _dev(e2s_np)
        for t in range(8):
            say("fused decode, small shape:", name, "token", t)
            xn = synthetic.activations(wl, 1, 900 + t)
            x = _dev(xn)
            B.moe_layer_forward(shape, x, 1, wr, None, e2s, tiny.slots, a.ids, a.w, a.y,
                                a.cold_count, a.cold_routes, a.ws)
            B.moe_route(shape, x, 1, wr, None, b.ids, b.w, b.ws)
            B.moe_experts_forward(shape, x, 1, b.ids, b.w, e2s, tiny.slots, b.y, b.cold_count,
                                  b.cold_routes, b.ws)
            torch.cuda.synchronize()
            no_device_errors(a.ws, b.ws)
            assert torch.equal(a.ids[:1], b.ids[:1]) and torch.equal(a.w[:1], b.w[:1])
            paths_agree(a.y[:1].cpu().numpy(), b.y[:1].cpu().numpy(), name)
            _, ids_ref, w_ref = compare_routes(a.ids[:1].cpu().numpy(), a.w[:1].cpu().numpy(),
                                               O.router_logits(xn, tiny.wr), wl.top_k)
            ref = O.layer_forward(xn, ids_ref, w_ref, tiny.experts, e2s_np)
            cc = int(a.cold_count.item())
            assert cc == len(ref["cold_routes"])
            if name == "all cold":
                assert not a.y[:1].any()
            else:
                close_enough(a.y[:1].cpu().numpy(), ref["y_hot"], f"fused small {name} {t}")
    for lay in (tiny, gptoss):
        shp = lay.shape
        w_dev = _dev(lay.wr)
        T = 4
        xs = [_dev(synthetic.activations(lay.wl, 1, 950 + t)) for t in range(T)]
        bufs = [L.Buffers(shp, 1) for _ in range(T)]
        ws = L.Buffers(shp, 1).ws  # one workspace shared by the calls, as in a layer loop

        def calls(stream=None):
            for t in range(T):
                kw = {} if stream is None else {"stream": stream}
                B.moe_layer_forward(shp, xs[t], 1, w_dev, None, None, lay.slots, bufs[t].ids,
                                    bufs[t].w, bufs[t].y, None, None, ws, **kw)

        say("fused graph:", lay.wl.name, "eager reference")
        calls()
        torch.cuda.synchronize()
        y_eager = [bf.y[:1].clone() for bf in bufs]
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                calls(s)
        torch.cuda.synchronize()
        for rep in range(3):
            say("fused graph:", lay.wl.name, "replay", rep)
            for bf in bufs:
                bf.y.zero_()
            g.replay()
            torch.cuda.synchronize()
            for t in range(T):
                assert torch.equal(bufs[t].y[:1], y_eager[t]), (lay.wl.name, rep, t)
            no_device_errors(ws)
            calls()  # eager calls on the same workspace between the replays
            torch.cuda.synchronize()


def test_layer_forward_residual_equals_layer_plus_residual(gptoss, tiny):
    """moe_layer_forward_residual == moe_layer_forward + moe_residual_bf16, bitwise, on the fused
    one-token path, the GEMV path and the grouped GEMM path, in place and into another buffer."""
    for lay, Ms in ((gptoss, (1, 3)), (tiny, (64, 130))):
        wl, shape = lay.wl, lay.shape
        wr = _dev(lay.wr)
        for M in Ms:
            say("layer_forward_residual:", wl.name, "M =", M)
            xn = synthetic.activations(wl, M, 1300 + M)
            a, b = L.Buffers(shape, M), L.Buffers(shape, M)
            x_ref = _dev(xn)
            B.moe_layer_forward(shape, x_ref, M, wr, None, None, lay.slots, a.ids, a.w, a.y,
                                a.cold_count, a.cold_routes, a.ws)
            nxt_ref = torch.zeros_like(x_ref)
            B.moe_residual_bf16(x_ref, a.y, nxt_ref, M * wl.hidden)
            x_sep = _dev(xn)
            nxt = torch.zeros_like(x_sep)
            B.moe_layer_forward_residual(shape, x_sep, M, wr, None, None, lay.slots, b.ids, b.w, b.y,
                                         b.cold_count, b.cold_routes, nxt, b.ws)
            torch.cuda.synchronize()
            no_device_errors(a.ws, b.ws)
            assert torch.equal(a.y[:M], b.y[:M]) and torch.equal(nxt_ref, nxt)
            assert torch.equal(x_sep, x_ref)  # the input is left alone
            x_in = _dev(xn)
            B.moe_layer_forward_residual(shape, x_in, M, wr, None, None, lay.slots, b.ids, b.w, b.y,
                                         b.cold_count, b.cold_routes, x_in, b.ws)
            torch.cuda.synchronize()
            assert torch.equal(a.y[:M], b.y[:M]) and torch.equal(x_in, nxt_ref)
    with pytest.raises(B.MoeError):
        B.moe_layer_forward_residual(gptoss.shape, x_ref, 1, wr, None, None, gptoss.slots, a.ids, a.w,
                                     a.y, None, None, None, a.ws)


def test_device_error_word_flags_bad_ids_and_slots(tiny):
    """Routes whose expert id lies outside [0, E) or whose expert maps to a slot outside
    [-1, S) are skipped like cold routes, and the call's device error word says so (read through
    moe_workspace_errors); the next good call on the same workspace clears it.  Covered: the
    route-table prologue (few routes), the top-k / bucketing kernel (more routes), the grouped
    GEMM path (M >= 64) and the fused one-token kernel (a bad map entry for a routed expert)."""
    wl = tiny.wl
    E, k, S = wl.n_experts, wl.top_k, wl.n_slots
    shape = tiny.shape
    for M in (3, 40, 64):
        say("device error word: M =", M)
        x = synthetic.activations(wl, M, 1500 + M)
        ids_ref, w_ref, _, _ = O.route(O.router_logits(x, tiny.wr), k)
        bad_e = int(ids_ref[0, 1])             # expert of route 1: its map entry is out of range
        e2s = np.arange(E, dtype=np.int32)
        e2s[bad_e] = S + 5
        ids = ids_ref.astype(np.int32).copy()
        ids[M - 1, 0] = E + 2                  # an id out of range
        buf = L.Buffers(shape, M)
        B.moe_experts_forward(shape, _dev(x), M, _dev(ids), _dev(w_ref.astype(np.float32)),
                              _dev(e2s), tiny.slots, buf.y, buf.cold_count, buf.cold_routes, buf.ws)
        torch.cuda.synchronize()
        assert device_errors(buf.ws) == B.MOE_DEVERR_BAD_ID | B.MOE_DEVERR_BAD_SLOT
        # reference: both kinds of bad route are cold (any expert whose map entry is -1 stands in)
        e2s_ref = e2s.copy()
        e2s_ref[bad_e] = -1
        ids_ref2 = ids.copy()
        ids_ref2[M - 1, 0] = bad_e
        ref = O.layer_forward(x, ids_ref2, w_ref, tiny.experts, e2s_ref)
        cc = int(buf.cold_count.item())
        assert cc == len(ref["cold_routes"])
        assert np.array_equal(buf.cold_routes[:cc].cpu().numpy(), ref["cold_routes"])
        close_enough(buf.y[:M].cpu().numpy(), ref["y_hot"], f"bad routes cold, M={M}")
        # a good call on the same workspace clears the word
        B.moe_experts_forward(shape, _dev(x), M, _dev(ids_ref.astype(np.int32)),
                              _dev(w_ref.astype(np.float32)), None, tiny.slots, buf.y, None, None,
                              buf.ws)
        torch.cuda.synchronize()
        assert device_errors(buf.ws) == 0
    say("device error word: fused one-token layer call with bad map entries")
    assert B.moe_layer_launches(shape, 1) == 1  # the router runs inside the fused kernel
    buf = L.Buffers(shape, 1)
    x = synthetic.activations(wl, 1, 1600)
    e2s = np.arange(E, dtype=np.int32)
    e2s[::2] = S + 1                           # every even expert: out of range
    B.moe_layer_forward(shape, _dev(x), 1, _dev(tiny.wr), None, _dev(e2s), tiny.slots, buf.ids,
                        buf.w, buf.y, buf.cold_count, buf.cold_routes, buf.ws)
    torch.cuda.synchronize()
    ids = buf.ids[:1].cpu().numpy()
    bad = bool((ids % 2 == 0).any())
    assert device_errors(buf.ws) == (B.MOE_DEVERR_BAD_SLOT if bad else 0)
    e2s_ref = e2s.copy()
    e2s_ref[::2] = -1
    ref = O.layer_forward(x, ids, oracle_weights_for(O.router_logits(x, tiny.wr), ids), tiny.experts,
                          e2s_ref)
    assert int(buf.cold_count.item()) == len(ref["cold_routes"])
    if np.linalg.norm(ref["y_hot"]) > 0:
        close_enough(buf.y[:1].cpu().numpy(), ref["y_hot"], "fused, bad map entries cold")
    else:
        assert not buf.y[:1].any()
    B.moe_layer_forward(shape, _dev(x), 1, _dev(tiny.wr), None, None, tiny.slots, buf.ids, buf.w,
                        buf.y, None, None, buf.ws)
    torch.cuda.synchronize()
    assert device_errors(buf.ws) == 0


def test_split_down_poisoned_workspace_flags_and_writes_nan(e512):
    """At 8 tokens on the E = 512 layer the down GEMV shares each row tile's hot experts between
    two workgroups, one handing its routes' rows to the other in words tagged with the tile's
    call id.  Against the oracle; then on a workspace whose poison word is set (what a lost
    hand-over leaves) the call gathers nothing, writes NaN rows and flags MOE_DEVERR_HANDOFF,
    without waiting; zero-filled again, the workspace gives bitwise the first result, twice.
    Before that, one workspace serves 16 tokens (the most that split), 17 (which do not) and 3,
    in turn, against the oracle."""
    wl = e512.wl
    counts = routed_counts(wl, 0, 256)
    slot_expert = popularity_placement(counts, wl.n_slots)
    e2s = np.full(wl.n_experts, -1, np.int32)
    e2s[slot_expert] = np.arange(wl.n_slots)
    shape = _shape(wl, wl.n_slots)
    slots = e512.slots_for(slot_expert)
    buf = L.Buffers(shape, 17)
    bias = synthetic.zipf_bias(wl)
    for M in (16, 17, 3):
        say("split down: one workspace, M =", M)
        x = synthetic.activations(wl, M, 60 + M)
        ids, w = run_route(shape, x, e512.wr, bias, M, buf)
        _, ids_ref, w_ref = compare_routes(ids, w, O.router_logits(x, e512.wr, bias), wl.top_k)
        y, _, _ = run_experts(shape, x, ids_ref, w_ref, e2s, slots, buf, M)
        close_enough(y, O.layer_forward(x, ids_ref, w_ref, e512.experts, e2s)["y_hot"],
                     f"split down M={M}")
    M = 8
    x = synthetic.activations(wl, M, 77)
    ids, w = run_route(shape, x, e512.wr, bias, M, buf)
    _, ids_ref, w_ref = compare_routes(ids, w, O.router_logits(x, e512.wr, bias), wl.top_k)
    say("split down: hand-over of rows between the two workgroups of each tile")
    y, cc, _ = run_experts(shape, x, ids_ref, w_ref, e2s, slots, buf, M)
    ref = O.layer_forward(x, ids_ref, w_ref, e512.experts, e2s)
    close_enough(y, ref["y_hot"], "split down M=8")
    say("split down: poisoned workspace")
    buf.ws.view(torch.int32)[7] = 1  # the poison word of the workspace header
    B.moe_experts_forward(shape, _dev(x), M, _dev(np.ascontiguousarray(ids_ref, np.int32)),
                          _dev(np.ascontiguousarray(w_ref, np.float32)), _dev(e2s), slots, buf.y,
                          buf.cold_count, buf.cold_routes, buf.ws)
    torch.cuda.synchronize()
    assert device_errors(buf.ws) == B.MOE_DEVERR_HANDOFF
    assert torch.isnan(buf.y[:M]).all()
    say("split down: zero-filled workspace")
    buf.ws.zero_()
    for _ in range(2):
        y2, cc2, _ = run_experts(shape, x, ids_ref, w_ref, e2s, slots, buf, M)
        assert cc2 == cc and np.array_equal(y2, y)


def test_split_down_one_workspace_for_two_shapes(e512):
    """One workspace serves two layer shapes whose few-token down GEMV both split their row
    tiles (E = 512, H = 2048 at 8 tokens; E = 64, H = 1024 at 4 tokens), alternately: every call
    against the oracle.  The handed-over rows sit at places that do not depend on the shape, so
    what one shape leaves behind is never taken for the other's."""
    wa = e512.wl
    counts = routed_counts(wa, 0, 256)
    slot_expert = popularity_placement(counts, wa.n_slots)
    e2s_a = np.full(wa.n_experts, -1, np.int32)
    e2s_a[slot_expert] = np.arange(wa.n_slots)
    shape_a = _shape(wa, wa.n_slots)
    slots_a = e512.slots_for(slot_expert)
    bias_a = synthetic.zipf_bias(wa)
    wb = synthetic.Workload("split_b", 7, 1024, 512, 64, 8, (4,), 64)
    lb = Layer(wb)
    shape_b = _shape(wb)
    size = max(B.moe_workspace_size(shape_a, 8), B.moe_workspace_size(shape_b, 4))
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    buf_a, buf_b = L.Buffers(shape_a, 8), L.Buffers(shape_b, 4)
    buf_a.ws = ws
    buf_b.ws = ws
    for i in range(5):
        if i % 2 == 0:
            M = 8
            say("two shapes, one workspace: E = 512, M = 8, call", i)
            x = synthetic.activations(wa, M, 300 + i)
            ids, w = run_route(shape_a, x, e512.wr, bias_a, M, buf_a)
            _, ids_ref, w_ref = compare_routes(ids, w, O.router_logits(x, e512.wr, bias_a), wa.top_k)
            y, _, _ = run_experts(shape_a, x, ids_ref, w_ref, e2s_a, slots_a, buf_a, M)
            close_enough(y, O.layer_forward(x, ids_ref, w_ref, e512.experts, e2s_a)["y_hot"],
                         f"shape A call {i}")
        else:
            M = 4
            say("two shapes, one workspace: E = 64, M = 4, call", i)
            x = synthetic.activations(wb, M, 400 + i)
            ids, w = run_route(shape_b, x, lb.wr, None, M, buf_b)
            _, ids_ref, w_ref = compare_routes(ids, w, O.router_logits(x, lb.wr), wb.top_k)
            y, _, _ = run_experts(shape_b, x, ids_ref, w_ref, None, lb.slots, buf_b, M)
            close_enough(y, O.layer_forward(x, ids_ref, w_ref, lb.experts)["y_full"], f"shape B call {i}")


@pytest.mark.parametrize("M", [1, 8])
def test_e512_chained_stack(e512, M):
    """Four stacked E = 512, k = 10 layers, each with its own router, Zipf prior and half-resident
    placement (from 256 warm-up tokens), chained on the GPU by moe_layer_forward_residual
    (x_{l+1} = bf16(x_l + y_l), in place, one workspace, no host step between the layers).  Every
    layer's input is recorded on the stream; afterwards each layer is checked against the oracle
    on that recorded input: ids, weights, cold report, y_hot, and the chained input of the next
    layer bit for bit."""
    wl = e512.wl
    NL = 4
    E, k, S, H = wl.n_experts, wl.top_k, wl.n_slots, wl.hidden
    shape = _shape(wl, S)
    layers = []
    for l in range(NL):
        say("chained stack: placing layer", l, "M =", M)
        wr = synthetic.router_weights(wl, l)
        bias = synthetic.zipf_bias(wl, l)
        slot_expert = popularity_placement(routed_counts(wl, l, 256), S)
        e2s = np.full(E, -1, np.int32)
        e2s[slot_expert] = np.arange(S, dtype=np.int32)
        # every layer's experts are the fixture's (byte copies), its routing is its own
        layers.append(dict(wr=wr, bias=bias, e2s=e2s, wr_d=_dev(wr), bias_d=_dev(bias),
                           e2s_d=_dev(e2s), slots=e512.slots_for(slot_expert)))
    x0 = synthetic.activations(wl, M, 77)
    xa = _dev(x0)
    ws = L.Buffers(shape, M).ws
    x_in = torch.zeros((NL + 1, M, H), dtype=torch.int16, device="cuda")
    ids = torch.zeros((NL, M, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((NL, M, k), dtype=torch.float32, device="cuda")
    y = torch.zeros((NL, M, H), dtype=torch.float32, device="cuda")
    cold = torch.zeros((NL, 1), dtype=torch.int32, device="cuda")
    cold_routes = torch.zeros((NL, M * k), dtype=torch.int32, device="cuda")
    errs = torch.full((NL,), -1, dtype=torch.int32, device="cuda")
    for l, ly in enumerate(layers):
        x_in[l].copy_(xa.view(M, H))
        B.moe_layer_forward_residual(shape, xa, M, ly["wr_d"], ly["bias_d"], ly["e2s_d"], ly["slots"],
                                     ids[l], w[l], y[l], cold[l], cold_routes[l], xa, ws)
        B.moe_workspace_errors(ws, errs[l:l + 1])
    x_in[NL].copy_(xa.view(M, H))
    torch.cuda.synchronize()
    assert errs.cpu().tolist() == [0] * NL
    xh = x_in.cpu().numpy().view(np.uint16)
    for l, ly in enumerate(layers):
        say("chained stack: checking layer", l)
        lg = O.router_logits(xh[l], ly["wr"], ly["bias"])
        ids_l = ids[l].cpu().numpy()
        compare_routes(ids_l, w[l].cpu().numpy(), lg, k)
        ref = O.layer_forward(xh[l], ids_l, oracle_weights_for(lg, ids_l), e512.experts, ly["e2s"])
        cc = int(cold[l].item())
        assert cc == len(ref["cold_routes"])
        assert np.array_equal(cold_routes[l, :cc].cpu().numpy(), ref["cold_routes"])
        yl = y[l].cpu().numpy()
        close_enough(yl, ref["y_hot"], f"chained stack layer {l} M={M}")
        xf = (xh[l].astype(np.uint32) << 16).view(np.float32)
        assert np.array_equal(xh[l + 1], synthetic.bf16_from_f32(xf + yl)), f"residual of layer {l}"


def test_slot_cache_pipeline_concurrent_with_poison():
    """The 8-slot GPT-OSS-20B-shaped layer over 160 decode steps as a real pipeline: the host
    policy observes routes D = 2 steps late through pinned memory and events (no device-wide
    synchronisation until the end), maps go up through a pinned ring, refills run on a copy
    stream after the event of the last step that read the victim slot, and the compute stream
    waits for a refill's event at the step it becomes visible.  Every evicted slot is first
    overwritten with 0xFF bytes on the copy stream (E8M0 255 is NaN, E2M1 0xF is -6): a kernel
    that read a slot while it was being refilled would put NaN into y.  Maps, plans and cold
    counts equal the oracle policy's replay bit for bit, and y_hot matches the oracle at every
    step."""
    wl = synthetic.WORKLOADS["gptoss20b_8slots"]
    steps, lag, D, R_MAP = 160, 3, 2, 8
    shape = _shape(wl, wl.n_slots)
    E, k, S, H = wl.n_experts, wl.top_k, wl.n_slots, wl.hidden
    say("concurrent pipeline: generating 32 experts")
    experts = synthetic.experts_canonical(wl, 0, range(E))
    bank_np = L.pack_bank(shape, experts)
    bank = L.pinned_bank(bank_np)
    init = np.argsort(synthetic.zipf_ranks(wl))[:S].astype(np.int32)
    slots = L.device_slots(bank_np, init, S)
    wr = synthetic.router_weights(wl)
    xs = np.concatenate([synthetic.activations(wl, 1, t) for t in range(steps)])
    biases = np.stack([synthetic.zipf_bias(wl, 0, synthetic.drift_shift(wl, t)) for t in range(steps)])
    xs_d, wr_d, biases_d = _dev(xs), _dev(wr), torch.from_numpy(biases).cuda()
    cache = B.MoeCache(shape, lag_steps=lag, initial_slot_expert=init)
    ws = L.Buffers(shape, 1).ws
    ids_d = torch.zeros((steps, k), dtype=torch.int32, device="cuda")
    w_d = torch.zeros((steps, k), dtype=torch.float32, device="cuda")
    y_d = torch.zeros((steps, H), dtype=torch.float32, device="cuda")
    cold_d = torch.zeros((steps, 1), dtype=torch.int32, device="cuda")
    cold_routes = torch.zeros((steps, k), dtype=torch.int32, device="cuda")
    errs_d = torch.full((steps,), -1, dtype=torch.int32, device="cuda")
    ids_h = torch.zeros((steps, k), dtype=torch.int32).pin_memory()
    maps_h = torch.zeros((R_MAP, E), dtype=torch.int32).pin_memory()
    maps_d = torch.zeros((R_MAP, E), dtype=torch.int32, device="cuda")
    comp, copy = torch.cuda.Stream(), torch.cuda.Stream()
    after = [B.event_create() for _ in range(steps)]
    waits, maps, plans, events = {}, [], [], list(after)
    torch.cuda.synchronize()
    for t in range(steps):
        obs = None
        if t - D >= 0:
            B.event_synchronize(after[t - D])  # this step's routes have reached pinned memory
            obs = ids_h[t - D].numpy().copy()
        m, plan, _ = cache.moe_cache_policy_step(t, obs)
        maps.append(m)
        plans.append(plan)
        r = t % R_MAP  # pinned slot r was last read by the upload of step t - R_MAP (done: R_MAP > D)
        maps_h[r].copy_(torch.from_numpy(m))
        for ev in waits.pop(t, []):
            B.stream_wait_event(comp, ev)
        with torch.cuda.stream(comp):
            maps_d[r].copy_(maps_h[r], non_blocking=True)
        B.moe_layer_forward(shape, xs_d[t], 1, wr_d, biases_d[t], maps_d[r], slots, ids_d[t], w_d[t],
                            y_d[t], cold_d[t], cold_routes[t], ws, stream=comp)
        B.moe_workspace_errors(ws, errs_d[t:t + 1], stream=comp)
        with torch.cuda.stream(comp):
            ids_h[t].copy_(ids_d[t], non_blocking=True)
        B.event_record(after[t], comp)
        if plan:
            B.stream_wait_event(copy, after[t])
            with torch.cuda.stream(copy):
                for (_, v, _, _) in plan:
                    slots[v].fill_(0xFF)  # poison: the slot holds NaN scales until its copy lands
            done = B.event_create()
            events.append(done)
            B.moe_slot_refill(shape, slots, bank, [p[0] for p in plan], [p[1] for p in plan], copy,
                              None, done)
            waits.setdefault(plan[0][3], []).append(done)
    torch.cuda.synchronize()
    cache.close()
    for ev in events:
        B.event_destroy(ev)
    assert errs_d.cpu().tolist() == [0] * steps
    # the oracle's replay of the same pipeline
    lg = O.router_logits(xs, wr, None) + biases.astype(np.float64)
    pol = SlotCachePolicy(E, S, init, policy=LRU, max_refills=2, lag=lag, max_pending=2)
    ids_gpu = ids_d.cpu().numpy()
    w_gpu = w_d.cpu().numpy()
    y_gpu = y_d.cpu().numpy()
    cold_gpu = cold_d.cpu().numpy()[:, 0]
    assert np.array_equal(ids_gpu, ids_h.numpy())
    excluded, _, _ = compare_routes(ids_gpu, w_gpu, lg, k)
    say("concurrent pipeline: near-tie tokens", excluded)
    # the policy replay observes the routes the pipeline observed (the oracle's, up to near-ties)
    w_own = oracle_weights_for(lg, ids_gpu)
    memo = {}
    n_refills = 0
    for t in range(steps):
        m_ref, plan_ref = pol.step(t, ids_gpu[t - D] if t - D >= 0 else None)
        assert np.array_equal(maps[t], m_ref), t
        assert plans[t] == plan_ref, t
        n_refills += len(plan_ref)
        ref = O.layer_forward(xs[t:t + 1], ids_gpu[t:t + 1], w_own[t:t + 1], experts, m_ref,
                              dense_memo=memo)
        assert cold_gpu[t] == len(ref["cold_routes"]), t
        assert np.all(np.isfinite(y_gpu[t])), f"step {t}: NaN in y (a poisoned slot was read)"
        if np.linalg.norm(ref["y_hot"]) > 0:
            close_enough(y_gpu[t:t + 1], ref["y_hot"], f"concurrent pipeline step {t}")
        else:
            assert not y_gpu[t].any(), t
    say(f"concurrent pipeline: {steps} steps, {n_refills} refills, hit rate "
        f"{pol.stats['hits'] / max(1, pol.stats['routes']):.3f}")
    assert n_refills > 20


@pytest.mark.parametrize("which,M", [("gptoss20b_8slots", 1), ("e512", 1), ("e512", 8)])
def test_hybrid_layer_hot_gpu_plus_cold_host_equals_full(which, M, e512):
    """moe_layer_forward_hybrid: the hot experts on the GPU, the cold routes on the host cores
    while the GPU runs, their sum added on the stream.  y equals, bit for bit, the GPU's hot-only
    output (moe_experts_forward on the same routes) plus the host's cold-only output
    (moe_cold_forward_host), and matches the oracle's full output (y_hot + y_cold = y_full)
    over consecutive calls on one staging."""
    if which == "e512":
        wl, experts, bank = e512.wl, e512.experts, e512.bank
        counts = routed_counts(wl, 0, 256)
        slot_expert = popularity_placement(counts, wl.n_slots)
        bias = synthetic.zipf_bias(wl)
    else:
        wl = synthetic.WORKLOADS[which]
        experts = synthetic.experts_canonical(wl, 0, range(wl.n_experts))
        bank = L.pack_bank(_shape(wl, wl.n_experts), experts)
        slot_expert = np.argsort(synthetic.zipf_ranks(wl))[:wl.n_slots].astype(np.int32)
        bias = synthetic.zipf_bias(wl)
    E, k, S, H = wl.n_experts, wl.top_k, wl.n_slots, wl.hidden
    shape = _shape(wl, S)
    e2s = np.full(E, -1, np.int32)
    e2s[slot_expert] = np.arange(S, dtype=np.int32)
    slots = L.device_slots(bank, slot_expert, S)
    pinned = L.pinned_bank(bank)
    wr = synthetic.router_weights(wl)
    staging = B.HybridStaging(shape, M)
    a, b = L.Buffers(shape, M), L.Buffers(shape, M)
    wr_d, bias_d, e2s_d = _dev(wr), _dev(bias), _dev(e2s)
    for t in range(3):
        say("hybrid layer:", which, "M =", M, "call", t)
        xn = synthetic.activations(wl, M, 1700 + t)
        x = _dev(xn)
        B.moe_layer_forward_hybrid(shape, x, M, wr_d, bias_d, e2s_d, e2s, slots, pinned.numpy(),
                                   a.ids, a.w, a.y, staging, a.ws, n_threads=8)
        B.moe_route(shape, x, M, wr_d, bias_d, b.ids, b.w, b.ws)
        B.moe_experts_forward(shape, x, M, b.ids, b.w, e2s_d, slots, b.y, b.cold_count, b.cold_routes, b.ws)
        torch.cuda.synchronize()
        no_device_errors(a.ws, b.ws)
        assert torch.equal(a.ids[:M], b.ids[:M]) and torch.equal(a.w[:M], b.w[:M])
        ids, w = a.ids[:M].cpu().numpy(), a.w[:M].cpu().numpy()
        y_cold = np.zeros((M, H), np.float32)
        B.moe_cold_forward_host(shape, bank, xn, M, ids, w, e2s, y_cold, 2)
        y_hot = b.y[:M].cpu().numpy()
        y = a.y[:M].cpu().numpy()
        assert np.array_equal(y, y_hot + y_cold)
        lg = O.router_logits(xn, wr, bias)
        compare_routes(ids, w, lg, k)
        ref = O.layer_forward(xn, ids, oracle_weights_for(lg, ids), experts, e2s)
        assert int(b.cold_count.item()) == len(ref["cold_routes"])
        close_enough(y, ref["y_full"], f"hybrid {which} M={M} call {t}")
        if len(ref["cold_routes"]):
            close_enough(y_cold, ref["y_cold"], f"hybrid {which} cold part")
    staging.close()


@pytest.mark.parametrize("serial,fused", [(False, False), (True, False), (False, True), (True, True)])
def test_device_cache_in_one_graph_matches_oracle_policy(serial, fused):
    """The GPU-resident slot cache over 256 decode steps of the 8-slot GPT-OSS-20B-shaped layer,
    captured as one HIP graph: per step, the policy kernel (observing the previous step's
    routes from device memory) publishes the map and plans <= 2 refills; the router, top-k and
    hot experts run with that map on the compute stream (as moe_route + moe_experts_forward, or
    as the one-launch moe_layer_forward); the copy kernel moves the planned
    experts from device-mapped pinned memory into their slots either on a side stream, after
    the previous step's layer (the last reader of the victims), with the layer of step t + L
    waiting for it (L = 3), or in the compute stream right after the policy kernel (L = 1).
    Maps, plans, counters and cold counts equal the oracle policy's replay bit for bit; y_hot
    matches the oracle at every step."""
    wl = synthetic.WORKLOADS["gptoss20b_8slots"]
    steps, lag = 256, (1 if serial else 3)
    E, k, S, H = wl.n_experts, wl.top_k, wl.n_slots, wl.hidden
    shape = _shape(wl, S)
    if fused:
        assert B.moe_layer_launches(shape, 1) == 1  # the router inside the one launch
    say("device cache: generating 32 experts")
    experts = synthetic.experts_canonical(wl, 0, range(E))
    bank_np = L.pack_bank(shape, experts)
    bank = L.pinned_bank(bank_np)
    init = np.argsort(synthetic.zipf_ranks(wl))[:S].astype(np.int32)
    slots = L.device_slots(bank_np, init, S)
    wr = synthetic.router_weights(wl)
    xs = np.concatenate([synthetic.activations(wl, 1, t) for t in range(steps)])
    biases = np.stack([synthetic.zipf_bias(wl, 0, synthetic.drift_shift(wl, t)) for t in range(steps)])
    xs_d, wr_d, biases_d = _dev(xs), _dev(wr), torch.from_numpy(biases).cuda()
    comp, copy = torch.cuda.Stream(), torch.cuda.Stream()
    cache = B.DeviceCache(shape, lag_steps=lag, initial_slot_expert=init, stream=comp)
    ws = L.Buffers(shape, 1).ws
    ids = torch.full((steps, k), -1, dtype=torch.int32, device="cuda")  # the last row: "none yet"
    w = torch.zeros((steps, k), dtype=torch.float32, device="cuda")
    y = torch.zeros((steps, H), dtype=torch.float32, device="cuda")
    maps = torch.zeros((steps, E), dtype=torch.int32, device="cuda")
    plans = torch.zeros((steps, 2 * B.REFILL_RECORD_BYTES), dtype=torch.uint8, device="cuda")
    nplan = torch.zeros((steps,), dtype=torch.int32, device="cuda")
    cold = torch.zeros((steps, 1), dtype=torch.int32, device="cuda")
    cold_routes = torch.zeros((steps, k), dtype=torch.int32, device="cuda")
    ev_plan = [B.event_create() for _ in range(steps)]
    ev_layer = [B.event_create() for _ in range(steps)]
    ev_copy = [B.event_create() for _ in range(steps)]
    torch.cuda.synchronize()

    def step(t):
        cache.step(ids[(t - 1) % steps], k, maps[t], plans[t], nplan[t:t + 1], stream=comp)
        B.event_record(ev_plan[t], comp)
        if serial:  # the refills land before this step's layer (their experts are not in its map)
            cache.copy(nplan[t:t + 1], plans[t], bank, slots, stream=comp)
        elif t - lag >= 0:
            B.stream_wait_event(comp, ev_copy[t - lag])  # refills visible now have landed
        if fused:
            B.moe_layer_forward(shape, xs_d[t], 1, wr_d, biases_d[t], maps[t], slots, ids[t], w[t],
                                y[t], cold[t], cold_routes[t], ws, stream=comp)
        else:
            B.moe_route(shape, xs_d[t], 1, wr_d, biases_d[t], ids[t], w[t], ws, stream=comp)
            B.moe_experts_forward(shape, xs_d[t], 1, ids[t], w[t], maps[t], slots, y[t], cold[t],
                                  cold_routes[t], ws, stream=comp)
        B.event_record(ev_layer[t], comp)
        if serial:
            return
        B.stream_wait_event(copy, ev_plan[t])
        if t >= 1:
            B.stream_wait_event(copy, ev_layer[t - 1])  # the victims' last readers are done
        cache.copy(nplan[t:t + 1], plans[t], bank, slots, stream=copy)
        B.event_record(ev_copy[t], copy)

    say("device cache: capturing", steps, "steps")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(comp):
        with torch.cuda.graph(g, stream=comp):
            for t in range(steps):
                step(t)
            if not serial:
                B.stream_wait_event(comp, ev_copy[steps - 1])  # join the copy stream
    torch.cuda.synchronize()
    say("device cache: replay")
    with torch.cuda.stream(comp):
        g.replay()
    torch.cuda.synchronize()
    no_device_errors(ws)
    st = cache.stats()
    ids_h, w_h, y_h = ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()
    maps_h, nplan_h, cold_h = maps.cpu().numpy(), nplan.cpu().numpy(), cold.cpu().numpy()[:, 0]
    plans_h = plans.cpu().numpy()
    lg = O.router_logits(xs, wr, None) + biases.astype(np.float64)
    excluded, _, _ = compare_routes(ids_h, w_h, lg, k)
    say("device cache: near-tie tokens", excluded)
    w_own = oracle_weights_for(lg, ids_h)
    pol = SlotCachePolicy(E, S, init, policy=LRU, max_refills=2, lag=lag, max_pending=2)
    memo, n_ref = {}, 0
    for t in range(steps):
        m_ref, plan_ref = pol.step(t, ids_h[t - 1:t] if t >= 1 else None)
        assert np.array_equal(maps_h[t], m_ref), t
        rec = plans_h[t].view(np.int32).reshape(2, 6)
        got = [(int(r[0]), int(r[1]), int(r[2]), int(r[4]) | (int(r[5]) << 32)) for r in rec[:nplan_h[t]]]
        assert got == plan_ref, (t, got, plan_ref)
        n_ref += len(plan_ref)
        ref = O.layer_forward(xs[t:t + 1], ids_h[t:t + 1], w_own[t:t + 1], experts, m_ref, dense_memo=memo)
        assert cold_h[t] == len(ref["cold_routes"]), t
        if np.linalg.norm(ref["y_hot"]) > 0:
            close_enough(y_h[t:t + 1], ref["y_hot"], f"device cache step {t}")
        else:
            assert not y_h[t].any(), t
    assert st == pol.stats, (st, pol.stats)
    say(f"device cache: {steps} steps in one graph, {n_ref} refills, hit rate "
        f"{st['hits'] / max(1, st['routes']):.3f}")
    assert n_ref > 20
    for ev in ev_plan + ev_layer + ev_copy:
        B.event_destroy(ev)


@pytest.mark.parametrize("M,n_slots", [(512, 48), (512, 256), (8, 8)])
def test_staged_prefill_matches_oracle(M, n_slots):
    """moe_layer_forward_staged on the E = 512, k = 10 layer with every expert in pinned host
    memory only: the touched experts are copied once into a staging slot array and the expert
    kernels (the grouped GEMMs at M = 512, the GEMVs at M = 8) run on it, in one pass when they
    fit and otherwise in double-buffered passes whose copies overlap the previous pass.  Every
    token matches the oracle's full output; a one-pass call equals moe_layer_forward over all
    experts resident bit for bit (slot numbering does not change the arithmetic)."""
    wl = synthetic.WORKLOADS["e512_prefill"]
    E, k, H = wl.n_experts, wl.top_k, wl.hidden
    shape = _shape(wl, E)
    say("staged prefill: experts, M =", M, "staging slots =", n_slots)
    experts = synthetic.experts_canonical(wl, 0, range(E))
    bank_np = L.pack_bank(shape, experts)
    pinned = L.pinned_bank(bank_np)
    wr, bias = synthetic.router_weights(wl), synthetic.zipf_bias(wl)
    x = synthetic.activations(wl, M, 31)
    st = B.PrefillStaging(shape, M, n_slots)
    a = L.Buffers(shape, M)
    results = []
    for rep in range(2):  # the second call reuses the staging
        a.y.fill_(3.0)
        nt, npass = B.moe_layer_forward_staged(shape, _dev(x), M, _dev(wr), _dev(bias), pinned, a.ids,
                                               a.w, a.y, st, a.ws)
        torch.cuda.synchronize()
        no_device_errors(a.ws)
        say(f"staged prefill: {nt} touched experts in {npass} passes")
        assert (npass == 1) == (nt <= n_slots)
        results.append(a.y[:M].clone())
    assert torch.equal(results[0], results[1])
    ids = a.ids[:M].cpu().numpy()
    lg = O.router_logits(x, wr, bias)
    compare_routes(ids, a.w[:M].cpu().numpy(), lg, k)
    assert nt == len(np.unique(ids))
    ref = O.layer_forward(x, ids, oracle_weights_for(lg, ids), experts)
    rel = close_enough(results[0].cpu().numpy(), ref["y_full"], f"staged prefill M={M} slots={n_slots}")
    say(f"staged prefill: rel-L2 {rel:.3e}")
    if npass == 1:
        b = L.Buffers(shape, M)
        B.moe_layer_forward(shape, _dev(x), M, _dev(wr), _dev(bias), None, L.device_slots(bank_np),
                            b.ids, b.w, b.y, None, None, b.ws)
        torch.cuda.synchronize()
        if M == 1:
            paths_agree(b.y[:M].cpu().numpy(), results[0].cpu().numpy(), "staged one pass")
        else:
            assert torch.equal(b.y[:M], results[0])
    st.close()


def test_device_cache_state_copy_is_a_checkpoint():
    """The GPU-resident cache's state is plain device memory: a copy taken at step t0 and written
    back replays steps t0.. with bit-identical maps, plans and counters, and matches the host
    policy restored from its own checkpoint at t0."""
    E, S, k = 32, 8, 4
    shape = B.make_shape(256, 512, E, k, S)
    init = np.arange(S, dtype=np.int32)
    cfg = dict(policy=B.MOE_POLICY_LFRU, max_refills_per_step=2, lag_steps=2, max_pending=3,
               decay_period=8)
    dc = B.DeviceCache(shape, initial_slot_expert=init, **cfg)
    host = B.MoeCache(shape, initial_slot_expert=init, **cfg)
    rng = np.random.default_rng(31)
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    T, t0 = 96, 50
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    obs = torch.from_numpy(ids).cuda()
    maps = torch.zeros((T, E), dtype=torch.int32, device="cuda")
    plans = torch.zeros((T, 2 * B.REFILL_RECORD_BYTES), dtype=torch.uint8, device="cuda")
    nplan = torch.zeros(T, dtype=torch.int32, device="cuda")

    def run(t_from):
        for t in range(t_from, T):
            dc.step(obs[t], k, maps[t], plans[t], nplan[t:t + 1])
        torch.cuda.synchronize()
        return maps[t_from:].cpu().numpy(), nplan[t_from:].cpu().numpy(), plans[t_from:].cpu().numpy()

    say("device cache checkpoint: first run")
    for t in range(t0):
        dc.step(obs[t], k, maps[t], plans[t], nplan[t:t + 1])
        host.moe_cache_policy_step(t, ids[t:t + 1])
    torch.cuda.synchronize()
    snap = dc.state.clone()
    host_snap = host.moe_cache_save()
    m1, n1, p1 = run(t0)
    stats1 = dc.stats()
    say("device cache checkpoint: replay from the copy")
    dc.state.copy_(snap)
    m2, n2, p2 = run(t0)
    assert np.array_equal(m1, m2) and np.array_equal(n1, n2)
    for i in range(T - t0):  # the planned records (unused record bytes are not written)
        nb = int(n1[i]) * B.REFILL_RECORD_BYTES
        assert np.array_equal(p1[i, :nb], p2[i, :nb]), i
    assert dc.stats() == stats1
    # the host policy restored at t0 plans the same maps
    host2 = B.MoeCache(shape)
    host2.moe_cache_restore(host_snap)
    for t in range(t0, T):
        m, plan, _ = host2.moe_cache_policy_step(t, ids[t:t + 1])
        assert np.array_equal(m, m1[t - t0]), t
        assert len(plan) == int(n1[t - t0]), t
    host.close()
    host2.close()


def test_many_routes_fall_back_to_the_grouped_path():
    """Below 64 tokens, a call whose down partial rows would not fit the GEMV kernel's LDS (here
    k = 32 routes per token, I = 1280 split in two K parts: 40 x 32 routes) runs the grouped
    kernels, and matches the oracle."""
    wl = synthetic.Workload("many_routes", 7, 256, 1280, 64, 32, (40,), 64)
    shape = B.make_shape(wl.hidden, wl.inter, wl.n_experts, wl.top_k, wl.n_slots)
    M = 40
    assert B.moe_layer_launches(shape, M) == 5
    assert B.moe_layer_launches(shape, 8) == 4
    experts = synthetic.experts_canonical(wl, 0, range(wl.n_experts))
    slots = L.device_slots(L.pack_bank(shape, experts))
    wr = synthetic.router_weights(wl)
    buf = L.Buffers(shape, M)
    for m in (M, 8):
        say("many routes: M =", m)
        x = synthetic.activations(wl, m, m)
        B.moe_layer_forward(shape, _dev(x), m, _dev(wr), None, None, slots, buf.ids, buf.w, buf.y,
                            buf.cold_count, buf.cold_routes, buf.ws)
        torch.cuda.synchronize()
        no_device_errors(buf.ws)
        _, ids_ref, w_ref = compare_routes(buf.ids[:m].cpu().numpy(), buf.w[:m].cpu().numpy(),
                                           O.router_logits(x, wr), wl.top_k)
        close_enough(buf.y[:m].cpu().numpy(), O.layer_forward(x, ids_ref, w_ref, experts)["y_full"],
                     f"many routes M={m}")


@pytest.mark.parametrize("H", [320, 2880, 8192])
def test_router_token_groups(H):
    """The one-wave-per-row router requests the x rows of a group of tokens together: 8, 4 or 2
    tokens by the row's width (H = 320, 2880, 8192), then the smaller groups for the rest.  Every
    token count from 1 to 17 (each tail: 4 + 2 + 1, 2 + 1, ...) against the oracle's routes."""
    E, k = 64, 6
    wl = synthetic.Workload(f"router_groups_{H}", 31, H, 256, E, k, (17,), E)
    shape = B.make_shape(H, 256, E, k, E)
    wr = synthetic.router_weights(wl)
    wrd = _dev(wr)
    buf = L.Buffers(shape, 17)
    for M in list(range(1, 10)) + [15, 17]:
        say(f"router groups H={H} M={M}")
        x = synthetic.activations(wl, M, M)
        buf.ids.fill_(-1)
        B.moe_route(shape, _dev(x), M, wrd, None, buf.ids, buf.w, buf.ws)
        torch.cuda.synchronize()
        no_device_errors(buf.ws)
        compare_routes(buf.ids[:M].cpu().numpy(), buf.w[:M].cpu().numpy(), O.router_logits(x, wr), k)
