"""moe_layer_forward_noalloc (the layer call on the library's static scratch, for callers that
cannot allocate) against moe_layer_forward with a workspace, through the C ABI, on two calls
in a row of which the second is smaller, on the fused one-token path, the few-token GEMV path
(on the E = 512 layer with row tiles shared by two workgroups, whose handed-over rows sit in the
same static array as the other shapes' calls) and the grouped GEMM path."""
import numpy as np
import pytest
import torch

import synthetic
from expert_offloaded_routed_amd import binding as B
from expert_offloaded_routed_amd import layer as L

from gpu_common import device_errors, say

pytestmark = pytest.mark.gpu


def _dev(a):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _both(shape, x, M, wr, bias, e2s, slots):
    """The same call through both entry points; returns (with-workspace, noalloc) outputs."""
    k, H = shape.top_k, shape.hidden
    a = L.Buffers(shape, M)
    B.moe_layer_forward(shape, x, M, wr, bias, e2s, slots, a.ids, a.w, a.y, a.cold_count,
                        a.cold_routes, a.ws)
    ids = torch.full((M, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((M, k), -7.0, dtype=torch.float32, device="cuda")
    y = torch.full((M, H), -7.0, dtype=torch.float32, device="cuda")
    cc = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    cr = torch.full((M * k,), -7, dtype=torch.int32, device="cuda")
    err = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    B.moe_layer_forward_noalloc(shape, x, M, wr, bias, e2s, slots, ids, w, y, cc, cr, err)
    torch.cuda.synchronize()
    assert device_errors(a.ws) == 0
    assert int(err.item()) == 0
    n = int(a.cold_count.item())
    assert torch.equal(a.ids[:M], ids) and torch.equal(a.w[:M], w), M
    assert torch.equal(a.y[:M], y), M
    assert int(cc.item()) == n and torch.equal(a.cold_routes[:n], cr[:n]), M
    return y


@pytest.mark.parametrize("name,Ms", [("gptoss20b_decode", (3, 1)), ("tiny", (64, 5)),
                                       ("e512_verify_stack", (8, 4))])
def test_noalloc_matches_layer_forward(name, Ms):
    wl = synthetic.WORKLOADS[name]
    E = wl.n_experts
    shape = B.make_shape(wl.hidden, wl.inter, E, wl.top_k, E)
    experts = synthetic.experts_canonical(wl, 0, range(E))
    slots = L.device_slots(L.pack_bank(shape, experts))
    wr = _dev(synthetic.router_weights(wl))
    bias = _dev(synthetic.zipf_bias(wl))
    e2s_np = np.arange(E, dtype=np.int32)
    e2s_np[1::3] = -1
    for i, M in enumerate(Ms):  # the second call is the smaller one
        for e2s in (None, _dev(e2s_np)):
            say("noalloc:", name, "M =", M, "map", "identity" if e2s is None else "partly cold")
            x = _dev(synthetic.activations(wl, M, 2000 + 10 * i + M))
            y = _both(shape, x, M, wr, bias, e2s, slots)
            assert torch.isfinite(y).all()


def test_noalloc_rejects_calls_beyond_the_scratch():
    wl = synthetic.WORKLOADS["e512_prefill"]
    shape = B.make_shape(wl.hidden, wl.inter, wl.n_experts, wl.top_k, wl.n_experts)
    M = wl.tokens[0]
    assert B.moe_workspace_size(shape, M) > 8 << 20
    say("noalloc: an M = 512, E = 512 call is refused before any launch")
    with pytest.raises(B.MoeError) as ex:
        B.moe_layer_forward_noalloc(shape, 0x1000, M, 0x1000, None, None, 0x1000, 0x1000, 0x1000,
                                    0x1000, None, None, None)
    assert ex.value.status == B.MOE_ERR_WORKSPACE
    assert "static scratch" in str(ex.value)
