"""The routed-MoE layer, evaluated by its plain definition in float64.

Sources (page title, section):
  * MoE expert offload (xinfer docs), intro and "How it works": placement of experts in GPU
    slots never changes routing or the math; the expert GEMMs read slot tensors.
  * [CUDA/CPU] Add hybrid GPU/CPU expert offload for MoEPacked block-packed weights
    (ONNX Runtime PR), "Key Changes": an optional expert_to_slot map; routes whose slot is
    negative (cold) are skipped by the GPU kernel and accumulated elsewhere.
  * tinyserve -- MoE Expert Offloading for Consumer GPUs, "How it works": per-expert
    gate/up/down on native quantised weights; batched calls group tokens by expert.

Readings where the pages are silent:
  * routing is the standard top-k gate: softmax over all E router logits, keep the k largest
    (ties to the lower expert id), renormalise the kept probabilities to sum to 1;
  * the expert FFN is plain SwiGLU without bias: h = silu(W_gate x) * (W_up x), d = W_down h;
    h is an activation and is rounded to bf16 (round to nearest even) before W_down;
  * the combine adds w[m,j] * d[m,j] over j = 0..k-1 in ascending j; cold routes keep their
    routed weight (no renormalisation), so hot-only + cold-only = full output.
"""
from __future__ import annotations

import numpy as np

from . import formats


# ---------------------------------------------------------------------------------------------
# bfloat16 <-> float64
# ---------------------------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 (exact: the bits are the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_rne(a) -> np.ndarray:
    """Round float64 values to bfloat16, nearest with ties to even; returns uint16 bits.

    bfloat16 keeps 8 significant bits with fp32's exponent range: a finite value a = f * 2^e
    (0.5 <= |f| < 1) is rounded to a multiple of 2^(e-8), but never finer than the smallest
    subnormal step 2^-133.  Results beyond the largest finite value become infinities.
    """
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)
    q = np.maximum(e.astype(np.int64) - 8, -133)
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.round(np.ldexp(a, -q))  # numpy rounds halves to even
        v = np.ldexp(r, q)
        v32 = v.astype(np.float32)  # exact for representable values; overflow -> inf
    bits = (v32.view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(np.isnan(a), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


# ---------------------------------------------------------------------------------------------
# Router, softmax, top-k, renormalise
# ---------------------------------------------------------------------------------------------
def router_logits(x_bits, w_router_bits, bias=None) -> np.ndarray:
    """l[m, e] = sum_h x[m, h] * W_r[e, h] + b[e], in float64.  x [M, H], W_r [E, H] bf16."""
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_router_bits)
    l = x @ w.T
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float64)[None, :]
    return l


def softmax(l: np.ndarray) -> np.ndarray:
    """Row softmax over all experts: exp(l - max) / sum exp(l - max)."""
    z = np.exp(l - l.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def route(logits: np.ndarray, k: int):
    """Softmax -> top-k -> renormalise.

    Returns ids int32 [M, k] (by probability descending, ties to the lower id), weights
    float64 [M, k] (the kept probabilities divided by their sum), the boundary gap
    p_(k) - p_(k+1) per token (inf when k == E) and the adjacent gaps inside the top-k
    [M, k-1] (used to recognise near-ties whose order or membership may legitimately differ).
    """
    p = softmax(np.asarray(logits, dtype=np.float64))
    M, E = p.shape
    ids = np.empty((M, k), dtype=np.int32)
    w = np.empty((M, k), dtype=np.float64)
    gap_k = np.empty(M, dtype=np.float64)
    inner = np.empty((M, max(k - 1, 0)), dtype=np.float64)
    for m in range(M):
        order = np.lexsort((np.arange(E), -p[m]))  # primary: p descending; secondary: id
        sel = order[:k]
        ids[m] = sel
        ps = p[m, sel]
        w[m] = ps / ps.sum()
        gap_k[m] = ps[-1] - p[m, order[k]] if k < E else np.inf
        inner[m] = ps[:-1] - ps[1:]
    return ids, w, gap_k, inner


# ---------------------------------------------------------------------------------------------
# Expert FFN and combine
# ---------------------------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def dequantize_expert(expert: dict) -> dict:
    """Canonical expert (gate/up [I,H], down [H,I]) -> float64 matrices.  The dict's "format"
    (absent: MXFP4) selects the decode (oracle.formats)."""
    return {name: formats.dequantize_matrix(expert, name) for name in ("gate", "up", "down")}


def expert_ffn(x: np.ndarray, dense: dict):
    """One expert on token rows x float64 [n, H]: returns (h_bits uint16 [n, I], d float64 [n, H])."""
    g = x @ dense["gate"].T
    u = x @ dense["up"].T
    h_bits = f64_to_bf16_rne(silu(g) * u)
    d = bf16_to_f64(h_bits) @ dense["down"].T
    return h_bits, d


def layer_forward(x_bits, ids, w, experts, expert_to_slot=None, dense_memo=None):
    """The expert half of the layer for given routes.

    x_bits uint16 [M, H]; ids int [M, k]; w float [M, k]; ``experts`` maps an expert id to
    its canonical MXFP4 dict (a list or a callable); expert_to_slot int [E] or None (all hot).
    ``dense_memo``: an optional dict that keeps each expert's dequantised matrices between
    calls (a cache of dequantize_expert, for long runs over the same experts).
    Returns a dict with y_hot, y_cold, y_full float64 [M, H], h_bits uint16 [M, k, I] and
    cold_routes (flat indices m*k + j, ascending).
    """
    x = bf16_to_f64(x_bits)
    ids = np.asarray(ids)
    w = np.asarray(w, dtype=np.float64)
    M, k = ids.shape
    H = x.shape[1]
    get = experts if callable(experts) else (lambda e: experts[e])
    hot = np.ones((M, k), dtype=bool)
    if expert_to_slot is not None:
        e2s = np.asarray(expert_to_slot)
        hot = e2s[ids] >= 0
    d = np.zeros((M, k, H), dtype=np.float64)
    h_bits = None
    for e in np.unique(ids):
        rows = np.argwhere(ids == e)  # (m, j) pairs routed to e
        if dense_memo is not None and int(e) in dense_memo:
            dense = dense_memo[int(e)]
        else:
            dense = dequantize_expert(get(int(e)))
            if dense_memo is not None:
                dense_memo[int(e)] = dense
        hb, de = expert_ffn(x[rows[:, 0]], dense)
        if h_bits is None:
            h_bits = np.zeros((M, k, hb.shape[1]), dtype=np.uint16)
        h_bits[rows[:, 0], rows[:, 1]] = hb
        d[rows[:, 0], rows[:, 1]] = de
    y_hot = np.zeros((M, H))
    y_cold = np.zeros((M, H))
    y_full = np.zeros((M, H))
    for m in range(M):
        for j in range(k):  # ascending j: the order of the deterministic combine
            term = w[m, j] * d[m, j]
            y_full[m] += term
            if hot[m, j]:
                y_hot[m] += term
            else:
                y_cold[m] += term
    cold_routes = np.flatnonzero(~hot.reshape(-1)).astype(np.int32)
    return {"y_hot": y_hot, "y_cold": y_cold, "y_full": y_full, "h_bits": h_bits,
            "cold_routes": cold_routes, "hot": hot}


# ---------------------------------------------------------------------------------------------
# Route buckets (group tokens by expert)
# ---------------------------------------------------------------------------------------------
def buckets(ids, n_experts: int):
    """counts[e] = routes to e; offsets = exclusive scan over ascending e (offsets[E] = M*k);
    perm lists the flat route indices m*k + j grouped by expert, ascending inside a bucket."""
    flat = np.asarray(ids).reshape(-1)
    counts = np.zeros(n_experts, dtype=np.int32)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    perm = np.empty(flat.size, dtype=np.int32)
    cursor = offsets[:-1].copy()
    for r, e in enumerate(flat):
        perm[cursor[e]] = r
        cursor[e] += 1
    return counts, offsets, perm
