"""Shared helpers of the GPU parity tests (not collected: no test_ prefix)."""
from __future__ import annotations

import sys

import numpy as np

import synthetic
from oracle import layer as O

REL_L2 = 1e-3        # rel-L2 bound on weights and outputs
MAX_ABS = 2e-2       # max-abs bound, relative to max |ref|
NEAR_TIE = 1e-6      # oracle probability gap under which top-k membership/order may differ


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device_errors(ws, stream=None):
    """The device error word of the last call on workspace ``ws``, read through the C ABI."""
    import torch

    from expert_offloaded_routed_amd import binding as B
    flags = torch.full((1,), -1, dtype=torch.int32, device=ws.device)
    B.moe_workspace_errors(ws, flags, stream=stream)
    torch.cuda.synchronize()
    return int(flags.item())


def no_device_errors(*workspaces):
    for ws in workspaces:
        f = device_errors(ws)
        assert f == 0, f"device error word {f:#x}"


def close_enough(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(got - ref) / nref if nref > 0 else np.linalg.norm(got)
    mx = np.abs(ref).max() if ref.size else 0.0
    mad = np.abs(got - ref).max() if ref.size else 0.0
    assert np.all(np.isfinite(got)), what
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e} > {REL_L2}"
    assert mad <= MAX_ABS * mx + 1e-30, f"{what}: max-abs {mad:.3e} > {MAX_ABS} * {mx:.3e}"
    return rel


PATH_REL_L2 = 1e-4   # two GPU paths of the same call (different matrix-core grouping)


def paths_agree(a, b, what=""):
    """Outputs of two GPU paths of one call: both deterministic, summed in different groupings
    on the matrix cores, so equal to well within the oracle bar (rel-L2 PATH_REL_L2)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, what
    nb = np.linalg.norm(b)
    rel = np.linalg.norm(a - b) / nb if nb > 0 else np.linalg.norm(a)
    assert rel <= PATH_REL_L2, f"{what}: paths differ by rel-L2 {rel:.3e}"
    return rel


def compare_routes(ids_gpu, w_gpu, logits_ref, k):
    """Top-k ids bit-exact except near-ties; weights within tolerance.  Returns #near-tie tokens."""
    ids_ref, w_ref, gap_k, inner = O.route(logits_ref, k)
    M = ids_ref.shape[0]
    excluded = 0
    got_w, ref_w = [], []
    for m in range(M):
        if gap_k[m] < NEAR_TIE:
            excluded += 1
            # any valid answer: the chosen set's weakest member is tied with the boundary
            p = O.softmax(logits_ref[m:m + 1])[0]
            chosen = set(int(v) for v in ids_gpu[m])
            assert len(chosen) == k
            assert min(p[list(chosen)]) >= np.sort(p)[::-1][k] - NEAR_TIE
            continue
        g = [int(v) for v in ids_gpu[m]]
        r = [int(v) for v in ids_ref[m]]
        assert set(g) == set(r), (m, g, r)
        for j in range(k):
            if g[j] != r[j]:  # only adjacent near-tied pairs may swap
                jj = r.index(g[j])
                lo = min(j, jj)
                assert abs(jj - j) == 1 and inner[m, lo] < NEAR_TIE, (m, g, r)
        order = np.argsort(ids_gpu[m])
        got_w.append(np.asarray(w_gpu[m])[order])
        ref_w.append(w_ref[m][np.argsort(ids_ref[m])])
    if got_w:
        close_enough(np.array(got_w), np.array(ref_w), "topk_w")
    return excluded, ids_ref, w_ref


def oracle_weights_for(logits_ref, ids):
    """The oracle's renormalised weights of the given routes (softmax over all experts, the
    chosen probabilities divided by their sum): for recomputing a token's output with the GPU's
    own top-k set, which may legitimately differ from the oracle's on a near-tie."""
    p = O.softmax(np.asarray(logits_ref, dtype=np.float64))
    ids = np.asarray(ids)
    ps = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    return ps / ps.sum(axis=1, keepdims=True)


def routed_counts(wl, layer, n_tokens, shift=0, warmup=True):
    """Oracle route counts over n_tokens warm-up tokens (M=1 steps) -> popularity ranking."""
    wr = synthetic.router_weights(wl, layer)
    bias = synthetic.zipf_bias(wl, layer, shift)
    x = np.concatenate([synthetic.activations(wl, 1, t, layer, warmup=warmup) for t in range(n_tokens)])
    ids, _, _, _ = O.route(O.router_logits(x, wr, bias), wl.top_k)
    return np.bincount(ids.reshape(-1), minlength=wl.n_experts)


def popularity_placement(counts, n_slots):
    """Experts ranked by (count desc, id asc); the top n_slots go to slots 0..n_slots-1."""
    order = sorted(range(len(counts)), key=lambda e: (-counts[e], e))
    return np.array(order[:n_slots], dtype=np.int32)
