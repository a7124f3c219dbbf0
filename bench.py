#!/usr/bin/env python3
"""Benchmark: routed-MoE layer decode on one MI355X.

Workload (default): GPT-OSS-20B-shaped layer -- hidden = intermediate = 2880, E = 32 MXFP4
experts, top_k = 4, M = 1 token per step, router logits biased by a Zipf(1.1) popularity
prior, every expert resident (identity expert_to_slot), a fresh activation every step.
One step = moe_layer_forward: router GEMV, softmax/top-k + resolve/bucketing, fused gate/up +
SiLU*up, down GEMV, ordered combine.  Steps are captured in a HIP graph.

Cache honesty: popular experts would otherwise stay in the 256 MB Infinity Cache between
steps, so step t reads copy t % R of the whole expert bank (R copies at distinct addresses,
reuse distance >= R * 52.9 MB).

Prints one JSON line: tok/s (= steps/s at M=1), the roofline of the dominant kernel (fused
gate/up) from HIP events on its own stream, and the CPU oracle's rate on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published peak


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=256)
    p.add_argument("--warmup", type=int, default=32)
    p.add_argument("--copies", type=int, default=16, help="distinct copies of the expert bank")
    p.add_argument("--kernel-reps", type=int, default=128, help="launches per kernel timing run")
    p.add_argument("--cpu-steps", type=int, default=12, help="oracle steps for cpu_baseline (0 = skip)")
    p.add_argument("--no-graph", action="store_true", help="time eager launches instead of a graph")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        return 2
    import torch

    import synthetic
    from expert_offloaded_routed_amd import binding as B
    from expert_offloaded_routed_amd import layer as L

    if not os.path.exists(B.LIB_PATH):
        from expert_offloaded_routed_amd import _build
        _build.build()
    B.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    wl = synthetic.WORKLOADS["gptoss20b_decode"]
    H, I, E, k = wl.hidden, wl.inter, wl.n_experts, wl.top_k
    shape = B.make_shape(H, I, E, k, E)
    t0 = time.time()
    experts = synthetic.experts_canonical(wl, 0, range(E))
    bank = L.pack_bank(shape, experts)
    img = bank.shape[1]
    print(f"[bench] generated + packed {E} experts ({bank.nbytes / 1e6:.1f} MB) in {time.time() - t0:.1f}s",
          file=sys.stderr, flush=True)
    R = max(1, args.copies)
    dev = torch.device("cuda:0")
    bank_d = torch.from_numpy(bank).to(dev)
    copies = torch.empty((R, E, img), dtype=torch.uint8, device=dev)
    for r in range(R):
        copies[r].copy_(bank_d)
    del bank_d
    wr = torch.from_numpy(synthetic.router_weights(wl).view(np.int16)).to(dev)
    bias = torch.from_numpy(synthetic.zipf_bias(wl)).to(dev)
    n_x = args.warmup + args.steps
    xs = torch.from_numpy(np.concatenate([synthetic.activations(wl, 1, t) for t in range(n_x)]).view(np.int16)).to(dev)
    ws_bytes = B.moe_workspace_size(shape, 1)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    ids = torch.zeros((n_x, k), dtype=torch.int32, device=dev)
    w = torch.zeros((n_x, k), dtype=torch.float32, device=dev)
    y = torch.zeros((n_x, H), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()

    def step(t):
        B.moe_layer_forward(shape, xs[t], 1, wr, bias, None, copies[t % R], ids[t], w[t], y[t], None,
                            None, ws, stream=stream)

    def capture(first, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for t in range(first, first + n):
                    step(t)
        return g

    # warm-up (also JIT/cache/first-touch)
    with torch.cuda.stream(stream):
        for t in range(args.warmup):
            step(t)
    torch.cuda.synchronize()
    if args.no_graph:
        g_timed = None
    else:
        g_warm = capture(0, max(1, args.warmup))
        g_timed = capture(args.warmup, args.steps)
        g_warm.replay()
    torch.cuda.synchronize()

    ev0, ev1 = B.event_create(timing=True), B.event_create(timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    B.event_record(ev0, stream)
    if g_timed is not None:
        with torch.cuda.stream(stream):
            g_timed.replay()
    else:
        with torch.cuda.stream(stream):
            for t in range(args.warmup, args.warmup + args.steps):
                step(t)
    B.event_record(ev1, stream)
    B.event_synchronize(ev1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_total = B.event_elapsed_ms(ev0, ev1)
    ms_step = ms_total / args.steps
    tok_s = args.steps / (ms_total / 1e3)

    # every step must have routed k distinct experts, all hot
    ids_h = ids[args.warmup:].cpu().numpy()
    assert np.all(np.sort(ids_h, axis=1)[:, 1:] != np.sort(ids_h, axis=1)[:, :-1])
    assert np.isfinite(y[args.warmup:].cpu().numpy()).all()
    exp_bytes = 13_219_200  # MXFP4 codes + E8M0 scales of gate, up and down of one expert
    assert exp_bytes == 3 * H * I // 2 + 3 * H * I // 32
    step_bytes = k * exp_bytes
    gbs_step = step_bytes / (ms_step * 1e-3) / 1e9

    # ---- dominant kernel: fused gate/up + SiLU*up, timed alone with HIP events on its stream
    gu_bytes = k * (2 * I * H // 2 + 2 * I * H // 32)  # algorithmic bytes per launch
    reps = args.kernel_reps
    t_last = args.warmup + args.steps - 1

    def kernel_graph(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for r in range(n):
                    fn(r)
        return g

    def time_graph(g, n):
        g.replay()  # warm
        torch.cuda.synchronize()
        B.event_record(ev0, stream)
        with torch.cuda.stream(stream):
            g.replay()
        B.event_record(ev1, stream)
        B.event_synchronize(ev1)
        return B.event_elapsed_ms(ev0, ev1) / n * 1e3  # us per launch

    g_gu = kernel_graph(lambda r: B.moe_experts_gateup(shape, xs[t_last], 1, ids[t_last], w[t_last], None,
                                                       copies[r % R], ws, stream=stream), reps)
    us_gu = time_graph(g_gu, reps)
    g_dn = kernel_graph(lambda r: B.moe_experts_down(shape, 1, ids[t_last], w[t_last], None, copies[r % R],
                                                     y[t_last], ws, stream=stream), reps)
    us_dn = time_graph(g_dn, reps)
    g_rt = kernel_graph(lambda r: B.moe_route(shape, xs[r % n_x], 1, wr, bias, ids[t_last], w[t_last], ws,
                                              stream=stream), reps)
    us_rt = time_graph(g_rt, reps)
    dn_bytes = k * (H * I // 2 + H * I // 32)
    gu_gbs = gu_bytes / (us_gu * 1e-6) / 1e9
    torch.cuda.synchronize()

    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        try:
            t = json.load(open(tfile))
            from expert_offloaded_routed_amd import _build
            if t.get("kernel_source_sha") == _build.kernel_source_sha():
                traffic = t.get("gateup_bytes_per_launch")
        except Exception:
            traffic = None

    # ---- CPU oracle on a bounded sample of the same workload
    cpu = None
    if args.cpu_steps > 0:
        from oracle import layer as O
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            cores = 1
        wr_h = synthetic.router_weights(wl)
        bias_h = synthetic.zipf_bias(wl)
        tc = time.perf_counter()
        for t in range(args.cpu_steps):
            x = synthetic.activations(wl, 1, t)
            oid, ow, _, _ = O.route(O.router_logits(x, wr_h, bias_h), k)
            O.layer_forward(x, oid, ow, experts)
        dt = time.perf_counter() - tc
        cpu = {"value": round(args.cpu_steps / dt, 4), "unit": "tok/s", "cores": cores, "kind": "oracle",
               "sample": f"{args.cpu_steps} decode steps (M=1) of the same layer: float64 router, "
                         f"top-k and dequantise-then-matmul of the 4 routed experts, {dt:.1f}s"}

    out = {
        "metric": "MoE-layer decode tok/s at M=1 + achieved HBM GB/s on expert weights vs peak",
        "value": round(tok_s, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights -> MXFP4, N(0,1) bf16 activations, Zipf(1.1) router prior)",
        "config": {"workload": "gptoss20b_decode", "hidden": H, "inter": I, "n_experts": E, "top_k": k,
                   "M": 1, "resident": "all (identity expert_to_slot)", "bank_copies": R,
                   "graph": not args.no_graph},
        "hbm_gbs_step": round(gbs_step, 1),
        "frac_peak_step": round(gbs_step / PEAK_HBM_GBS, 4),
        "expert_bytes_per_step": step_bytes,
        "kernels_us": {"route (router GEMV + top-k)": round(us_rt, 2),
                       "gateup (incl. route table)": round(us_gu, 2),
                       "down_combine (incl. route table)": round(us_dn, 2)},
        "down_gbs": round(dn_bytes / (us_dn * 1e-6) / 1e9, 1),
        "wall_s": round(wall, 4),
        "roofline": {"bound": "hbm", "kernel": "k_gateup (fused MXFP4 gate/up GEMV + SiLU*up)",
                     "achieved": round(gu_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": gu_bytes, "us_per_launch": round(us_gu, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
