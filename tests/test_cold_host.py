"""The cold routes on the host cores (moe_cold_forward_host, the CPU half of the hybrid layer)
against the oracle's cold-only output, on the CPU: no GPU is needed.  The oracle evaluates the
plain definition in float64; the host path decodes the same expert images the GPU slots hold and
accumulates in fp32."""
import numpy as np
import pytest

import synthetic
from expert_offloaded_routed_amd import binding as B
from expert_offloaded_routed_amd import layer as L
from oracle import layer as O

from gpu_common import close_enough


def _lib():
    import os
    if not os.path.exists(B.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return B.load()


@pytest.mark.parametrize("name,M,H,I,E,k", [("tiny", 5, 256, 512, 8, 2),
                                            ("e512_shape", 3, 2048, 512, 24, 10),
                                            ("odd_blocks", 2, 320, 480, 6, 3)])
def test_cold_routes_on_host_match_oracle(name, M, H, I, E, k):
    """I = 480 has 15 down blocks: a partial last K step of the down tiles."""
    _lib()
    import dataclasses
    wl = dataclasses.replace(synthetic.WORKLOADS["tiny"], name=name, hidden=H, inter=I, n_experts=E,
                             top_k=k, n_slots=E)
    shape = B.make_shape(H, I, E, k, E)
    experts = synthetic.experts_canonical(wl, 0, range(E))
    bank = L.pack_bank(shape, experts)
    rng = np.random.default_rng(len(name) + M)
    x = synthetic.activations(wl, M, 3)
    ids, w, _, _ = O.route(O.router_logits(x, synthetic.router_weights(wl)), k)
    for trial, frac in enumerate((0.5, 1.0, 0.0)):
        e2s = np.arange(E, dtype=np.int32)
        e2s[rng.random(E) < frac] = -1
        ref = O.layer_forward(x, ids, w, experts, e2s)
        y = np.full((M, H), 7.0, np.float32)
        B.moe_cold_forward_host(shape, bank, x, M, ids.astype(np.int32), w.astype(np.float32), e2s, y, 3)
        if np.linalg.norm(ref["y_cold"]) > 0:
            close_enough(y, ref["y_cold"], f"{name} cold-only output, trial {trial}")
        else:
            assert not y.any()
        # the same bits on one thread and on several
        y1 = np.empty_like(y)
        B.moe_cold_forward_host(shape, bank, x, M, ids.astype(np.int32), w.astype(np.float32), e2s, y1, 1)
        assert np.array_equal(y, y1)
    # no map: nothing is cold
    y = np.full((M, H), 7.0, np.float32)
    B.moe_cold_forward_host(shape, bank, x, M, ids.astype(np.int32), w.astype(np.float32), None, y, 2)
    assert not y.any()
