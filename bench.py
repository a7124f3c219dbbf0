#!/usr/bin/env python3
"""Benchmark: routed-MoE layer on one MI355X.

Default (the headline line): GPT-OSS-20B-shaped layer decode -- hidden = intermediate = 2880,
E = 32 MXFP4 experts, top_k = 4, M = 1 token per step, router logits biased by a Zipf(1.1)
popularity prior, every expert resident (identity expert_to_slot), a fresh activation every
step.  One step = moe_layer_forward: router GEMV, softmax/top-k + slot resolve + route table,
fused gate/up + SiLU*up, down GEMV + ordered combine.  The timed steps are one HIP graph.

Cache honesty: popular experts would otherwise stay in the 256 MB Infinity Cache between
steps, so step t reads copy t % R of the whole expert bank (R copies at distinct addresses,
reuse distance >= R * 52.9 MB).

Dominant kernel: the fused expert kernel (gate/up + SiLU*up, then down + ordered combine in one
launch; with MOE_DECODE_UNFUSED=1 the gate/up kernel of the two-launch path).  Its duration
comes from HIP events that moe_layer_forward_marked records on the launch stream at the stage
boundaries of the same steps, enqueued behind a spin kernel so that they run back to back;
achieved GB/s = its algorithmic bytes (the MXFP4 codes and scales of the 4 routed experts'
gate, up and down matrices; gate and up only for the gate/up kernel) / that duration.

Other workloads (one JSON line each, --workload):
  slots8    8 GPU slots for 32 experts, LRU refills (<= 2 per step) from pinned host memory on a
            side stream, drifting Zipf popularity: hit rate, hot-path tok/s, refill overlap.
  stack48   48 stacked E=512 layers (H=2048, I=512, k=10), 256 of 512 experts resident per layer
            by warm-up popularity, M in {1, 4, 8} (--tokens), residual chaining: tok/s.
  prefill   one E=512 layer, M=512 tokens, grouped GEMM on MFMA: GB/s, TFLOP/s.
  slots8dev the slots8 workload with the cache policy and the copies on the GPU, one graph.
  hybrid    8 static GPU slots, cold routes computed on the host cores.
  staged    the prefill layer with every expert in host memory, 48 staging slots.
  fate      next-layer prefetch predicted from the current layer's input: recall, hit rate.
  formats   the decode workload with bf16, block FP8 or NVFP4 experts (--format).
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

PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published peak
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published peak


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=256)
    p.add_argument("--warmup", type=int, default=32)
    p.add_argument("--workload", default="decode",
                   choices=["decode", "slots8", "slots8dev", "hybrid", "stack48", "prefill", "staged",
                            "fate", "formats"])
    p.add_argument("--format", default="nvfp4", choices=["bf16", "fp8_block", "nvfp4"],
                   help="formats: the experts' format")
    p.add_argument("--tokens", type=int, default=1, help="stack48: tokens per step (1, 4 or 8)")
    p.add_argument("--copies", type=int, default=16, help="distinct copies of the expert bank")
    p.add_argument("--stage-steps", type=int, default=256, help="marked steps for stage timing")
    p.add_argument("--enqueue-spin-cycles", type=float, default=2e8,
                   help="GPU cycles of the spin kernel that holds the stream while marked steps are enqueued")
    p.add_argument("--cpu-steps", type=int, default=40, help="oracle steps for cpu_baseline (0 = skip)")
    p.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="write profiles/traffic.json from two rocprofv3 counter runs of "
                        "--calibrate-copy-mb 256 (FETCH_SIZE, then WRITE_SIZE) and exit")
    p.add_argument("--calibrate-copy-mb", type=int, default=0,
                   help="after the run, copy a buffer of this many MiB device to device 4 times (a "
                        "plain copy kernel of known size, to scale HBM byte counters)")
    return p.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def setup():
    import torch

    from expert_offloaded_routed_amd import binding as B
    if not os.path.exists(B.LIB_PATH):
        from expert_offloaded_routed_amd import _build
        _build.build()
    B.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    return torch, B


def dev_bits(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def capture(torch, stream, fn, n):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                fn(i)
    return g


def time_graph(torch, B, stream, g):
    """GPU ms of one replay of g, from HIP events on its stream (after an untimed replay)."""
    ev0, ev1 = B.event_create(timing=True), B.event_create(timing=True)
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    B.event_record(ev0, stream)
    with torch.cuda.stream(stream):
        g.replay()
    B.event_record(ev1, stream)
    B.event_synchronize(ev1)
    ms = B.event_elapsed_ms(ev0, ev1)
    B.event_destroy(ev0)
    B.event_destroy(ev1)
    return ms


def cpu_cores():
    """Threads the oracle's numpy (BLAS) work runs on."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return 1


def nproc():
    try:
        return len(os.sched_getaffinity(0))
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(work, n, n1, per_unit, unit, sample):
    """Times the oracle: work(i) for i < n on the host's BLAS threads, then work(i) for i < n1 on
    one thread; value = per_unit / (seconds per work item)."""
    tc = time.perf_counter()
    for i in range(n):
        work(i)
    dt = (time.perf_counter() - tc) / n
    one = None
    if n1 > 0:
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(1):
                tc = time.perf_counter()
                for i in range(n1):
                    work(i)
                one = (time.perf_counter() - tc) / n1
        except Exception:
            one = None
    return {"value": round(per_unit / dt, 4), "unit": unit, "cores": cpu_cores(), "nproc": nproc(),
            "value_1core": round(per_unit / one, 4) if one else None, "kind": "oracle",
            "sample": f"{sample}: {n} items on {cpu_cores()} BLAS threads ({dt * n:.1f}s), "
                      f"{n1} on one thread"}


def stream_ceiling(torch, B, src, nbytes, stream, reps=64):
    """Read-streaming ceiling: moe_hbm_read_probe over nbytes windows of src (rotating, so that
    no window is cache-resident), GB/s of the average launch from HIP events."""
    total = src.numel()
    n_win = max(1, total // nbytes)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ev0, ev1 = B.event_create(timing=True), B.event_create(timing=True)
    for r in range(8):
        B.moe_hbm_read_probe(src[(r % n_win) * nbytes:], nbytes, sink, stream=stream)
    B.event_record(ev0, stream)
    for r in range(reps):
        B.moe_hbm_read_probe(src[(r % n_win) * nbytes:], nbytes, sink, stream=stream)
    B.event_record(ev1, stream)
    B.event_synchronize(ev1)
    us = B.event_elapsed_ms(ev0, ev1) * 1e3 / reps
    B.event_destroy(ev0)
    B.event_destroy(ev1)
    return nbytes / (us * 1e-6) / 1e9, us


# ---------------------------------------------------------------------------------------------
# Default: GPT-OSS-20B-shaped decode (the headline)
# ---------------------------------------------------------------------------------------------
def bench_decode(args):
    torch, B = setup()
    import synthetic
    from expert_offloaded_routed_amd import layer as L

    wl = synthetic.WORKLOADS["gptoss20b_decode"]
    H, I, E, k = wl.hidden, wl.inter, wl.n_experts, wl.top_k
    shape = B.make_shape(H, I, E, k, E)
    t0 = time.time()
    experts = synthetic.experts_canonical(wl, 0, range(E))
    bank = L.pack_bank(shape, experts)
    img = bank.shape[1]
    log(f"generated + packed {E} experts ({bank.nbytes / 1e6:.1f} MB) in {time.time() - t0:.1f}s")
    R = max(1, args.copies)
    bank_d = torch.from_numpy(bank).cuda()
    copies = torch.empty((R, E, img), dtype=torch.uint8, device="cuda")
    for r in range(R):
        copies[r].copy_(bank_d)
    del bank_d
    wr = dev_bits(torch, synthetic.router_weights(wl))
    bias = torch.from_numpy(synthetic.zipf_bias(wl)).cuda()
    n_x = args.warmup + args.steps
    xs = dev_bits(torch, np.concatenate([synthetic.activations(wl, 1, t) for t in range(n_x)]))
    ws = torch.zeros(B.moe_workspace_size(shape, 1), dtype=torch.uint8, device="cuda")
    ids = torch.zeros((n_x, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((n_x, k), dtype=torch.float32, device="cuda")
    y = torch.zeros((n_x, H), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()

    def step(t):
        B.moe_layer_forward(shape, xs[t], 1, wr, bias, None, copies[t % R], ids[t], w[t], y[t], None,
                            None, ws, stream=stream)

    with torch.cuda.stream(stream):
        for t in range(args.warmup):
            step(t)
    torch.cuda.synchronize()
    g_timed = capture(torch, stream, lambda i: step(args.warmup + i), args.steps)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ms_total = time_graph(torch, B, stream, g_timed)
    wall = time.perf_counter() - t_wall
    ms_step = ms_total / args.steps
    tok_s = args.steps / (ms_total / 1e3)

    # every step routed k distinct experts, all hot, and produced finite outputs
    ids_h = ids[args.warmup:].cpu().numpy()
    srt = np.sort(ids_h, axis=1)
    assert np.all(srt[:, 1:] != srt[:, :-1])
    assert np.isfinite(y[args.warmup:].cpu().numpy()).all()
    exp_bytes = 3 * H * I // 2 + 3 * H * I // 32  # MXFP4 codes + E8M0 scales, gate + up + down
    step_bytes = k * exp_bytes
    gu_bytes = k * (2 * I * H // 2 + 2 * I * H // 32)  # gate/up kernel, algorithmic bytes per launch

    # stage timing: the same steps as marked calls (events without a system fence at every stage
    # boundary, on the launch stream).  The stream first runs a bounded spin kernel long enough
    # for the host to enqueue every step, so the steps then run back to back and no host gap
    # falls inside a stage.  One untimed pass first.
    n_st = max(1, min(args.stage_steps, args.steps))
    marks = [[B.event_create(timing=True, system_fence=False) for _ in range(4)] for _ in range(n_st)]
    for rep in range(2):
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            torch.cuda._sleep(int(args.enqueue_spin_cycles))
            t_enq = time.perf_counter()
            for i in range(n_st):
                t = args.warmup + i
                B.moe_layer_forward_marked(shape, xs[t], 1, wr, bias, None, copies[t % R], ids[t], w[t],
                                           y[t], None, None, ws, marks[i], stream=stream)
            t_enq = time.perf_counter() - t_enq
    torch.cuda.synchronize()
    spin_ms = B.event_elapsed_ms(marks[0][0], marks[-1][3])
    log(f"stage timing: host enqueue {t_enq * 1e3:.1f} ms for {n_st} steps, GPU {spin_ms:.2f} ms")
    st = np.array([[B.event_elapsed_ms(m[j], m[j + 1]) for j in range(3)] for m in marks]) * 1e3
    span = np.array([B.event_elapsed_ms(m[0], m[3]) for m in marks]) * 1e3
    for m in marks:
        for e in m:
            B.event_destroy(e)
    us_rt, us_gu, us_dn = (float(v) for v in st.mean(axis=0))
    launches = B.moe_layer_launches(shape, 1)
    fused = launches <= 2
    if fused:  # marks[2] and marks[3] both follow the one expert launch
        dom_bytes, dom_us, dom_key = step_bytes, us_gu, "layer_decode_bytes_per_launch"
        dom_name = ("k_layer_decode (" + ("router GEMV, " if launches == 1 else "") +
                    "route table + MXFP4 gate/up GEMV + SiLU*up, then down GEMV + ordered combine, "
                    "one launch)")
        stages = ({"layer (router, route table, gate/up, down, combine: one launch)": round(us_gu, 2)}
                  if launches == 1 else
                  {"route (router GEMV)": round(us_rt, 2),
                   "experts (fused gate/up + down + combine)": round(us_gu, 2)})
    else:
        dom_bytes, dom_us, dom_key = gu_bytes, us_gu, "gateup_bytes_per_launch"
        dom_name = "k_gateup (route table + fused MXFP4 gate/up GEMV + SiLU*up)"
        stages = {"route (router GEMV)": round(us_rt, 2),
                  "gateup (route table + gate/up + SiLU*up)": round(us_gu, 2),
                  "down (down GEMV + ordered combine)": round(us_dn, 2)}
    dom_gbs = dom_bytes / (dom_us * 1e-6) / 1e9

    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        try:
            from expert_offloaded_routed_amd import _build
            t = json.load(open(tfile))
            if t.get("kernel_source_sha") == _build.kernel_source_sha():
                traffic = t.get(dom_key)
        except Exception:
            traffic = None

    # the read-streaming ceiling of a weight stream of the step's size, same launch shape
    ceil_gbs, ceil_us = stream_ceiling(torch, B, copies.view(-1), step_bytes, stream)
    log(f"read-streaming ceiling: {ceil_gbs:.0f} GB/s ({ceil_us:.2f} us per {step_bytes} B)")

    cpu = None
    if args.cpu_steps > 0:
        from oracle import layer as O
        wr_h = synthetic.router_weights(wl)
        bias_h = synthetic.zipf_bias(wl)

        near = set()

        def work(t):
            x = synthetic.activations(wl, 1, t)
            oid, ow, gap, _ = O.route(O.router_logits(x, wr_h, bias_h), k)
            if gap[0] < 1e-6:  # a near-tie: any valid top-k set is accepted for this token
                near.add(t)
            O.layer_forward(x, oid, ow, experts)
        cpu = cpu_baseline(work, args.cpu_steps, max(1, args.cpu_steps // 8), 1.0, "tok/s",
                           "decode steps (M=1) of the same layer: float64 router, top-k and "
                           "dequantise-then-matmul of the 4 routed experts")
        cpu["near_tie_tokens"] = len(near)

    gbs_step = step_bytes / (ms_step * 1e-3) / 1e9
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
                   "timed": "one HIP graph of the steps"},
        "hbm_gbs_step": round(gbs_step, 1),
        "frac_peak_step": round(gbs_step / PEAK_HBM_GBS, 4),
        "expert_bytes_per_step": step_bytes,
        "stage_us": stages,
        "step_us_marked_p50_p99": [round(float(np.percentile(span, 50)), 2),
                                  round(float(np.percentile(span, 99)), 2)],
        "wall_s": round(wall, 4),
        "roofline": {"bound": "hbm", "kernel": dom_name,
                     "achieved": round(dom_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": dom_bytes, "us_per_launch": round(dom_us, 3),
                     "launches_timed": n_st, "measured_ceiling_gbs": round(ceil_gbs, 1),
                     "frac_of_measured_ceiling": round(dom_gbs / ceil_gbs, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


# ---------------------------------------------------------------------------------------------
# slots8: 8 GPU slots, LRU refills from pinned host memory
# ---------------------------------------------------------------------------------------------
def bench_slots8(args):
    torch, B = setup()
    import synthetic
    from expert_offloaded_routed_amd import layer as L

    wl = synthetic.WORKLOADS["gptoss20b_8slots"]
    H, I, E, k, S = wl.hidden, wl.inter, wl.n_experts, wl.top_k, wl.n_slots
    shape = B.make_shape(H, I, E, k, S)
    experts = synthetic.experts_canonical(wl, 0, range(E))
    bank_np = L.pack_bank(shape, experts)
    bank = L.pinned_bank(bank_np)
    img = bank_np.shape[1]
    ranks = synthetic.zipf_ranks(wl)
    init = np.argsort(ranks)[:S].astype(np.int32)
    slots = L.device_slots(bank_np, init, S)
    wr = dev_bits(torch, synthetic.router_weights(wl))
    steps = args.steps
    n_x = args.warmup + steps
    xs = dev_bits(torch, np.concatenate([synthetic.activations(wl, 1, t) for t in range(n_x)]))
    biases = torch.from_numpy(np.stack([synthetic.zipf_bias(wl, 0, synthetic.drift_shift(wl, t))
                                        for t in range(n_x)])).cuda()
    comp = torch.cuda.Stream()
    copy = torch.cuda.Stream()

    # calibration: one refill batch (2 experts) on the copy stream
    e0, e1 = B.event_create(timing=True), B.event_create(timing=True)
    B.event_record(e0, copy)
    B.moe_slot_refill(shape, slots, bank, [int(init[0]), int(init[1])], [0, 1], copy, None, None)
    B.event_record(e1, copy)
    B.event_synchronize(e1)
    copy_ms = B.event_elapsed_ms(e0, e1)
    R_MAP = 64  # device copies of the expert map, reused round robin
    maps_d = torch.zeros((R_MAP, E), dtype=torch.int32, device="cuda")
    maps_h = torch.zeros((R_MAP, E), dtype=torch.int32).pin_memory()
    ids_h = torch.zeros((n_x, k), dtype=torch.int32).pin_memory()
    ids_d = torch.zeros((n_x, k), dtype=torch.int32, device="cuda")
    w_d = torch.zeros((n_x, k), dtype=torch.float32, device="cuda")
    y_d = torch.zeros((n_x, H), dtype=torch.float32, device="cuda")
    cold_d = torch.zeros((n_x,), dtype=torch.int32, device="cuda")
    cold_routes = torch.zeros((k,), dtype=torch.int32, device="cuda")
    ws = torch.zeros(B.moe_workspace_size(shape, 1), dtype=torch.uint8, device="cuda")

    def run(lag_steps, n_steps, timed):
        """The decode pipeline: host policy on ids read back D steps late, refills on the copy
        stream after the step that last read the victim slot, compute waits for a refill at the
        step it becomes visible."""
        cache = B.MoeCache(shape, lag_steps=lag_steps, initial_slot_expert=init)
        slots.copy_(L.device_slots(bank_np, init, S))
        D = 2
        after = [B.event_create() for _ in range(n_steps)]
        pre_t = [B.event_create(timing=True) for _ in range(n_steps)]
        post_t = [B.event_create(timing=True) for _ in range(n_steps)]
        cp0, cp1 = [], []
        waits = {}
        step_has_wait = np.zeros(n_steps, bool)
        stats = None
        torch.cuda.synchronize()
        tw = time.perf_counter()
        for t in range(n_steps):
            obs = None
            if t - D >= 0:
                B.event_synchronize(after[t - D])
                obs = ids_h[t - D].numpy()
            m, plan, stats = cache.moe_cache_policy_step(t, obs)
            B.event_record(pre_t[t], comp)
            for ev in waits.pop(t, []):
                B.stream_wait_event(comp, ev)
                step_has_wait[t] = True
            r = t % R_MAP
            maps_h[r].copy_(torch.from_numpy(m))
            with torch.cuda.stream(comp):
                maps_d[r].copy_(maps_h[r], non_blocking=True)
            B.moe_layer_forward(shape, xs[t], 1, wr, biases[t], maps_d[r], slots, ids_d[t], w_d[t], y_d[t],
                                cold_d[t:t + 1], cold_routes, ws, stream=comp)
            with torch.cuda.stream(comp):
                ids_h[t].copy_(ids_d[t], non_blocking=True)
            B.event_record(post_t[t], comp)
            B.event_record(after[t], comp)
            if plan:
                a, b = B.event_create(timing=True), B.event_create(timing=True)
                done = B.event_create()
                B.stream_wait_event(copy, after[t])
                B.event_record(a, copy)
                B.moe_slot_refill(shape, slots, bank, [p[0] for p in plan], [p[1] for p in plan], copy,
                                  None, done)
                B.event_record(b, copy)
                cp0.append(a)
                cp1.append(b)
                waits.setdefault(plan[0][3], []).append(done)
        torch.cuda.synchronize()
        wall = time.perf_counter() - tw
        res = {"wall_s": wall, "stats": stats,
               "copy_ms": [B.event_elapsed_ms(a, b) for a, b in zip(cp0, cp1)],
               "step_ms": np.array([B.event_elapsed_ms(a, b) for a, b in zip(pre_t, post_t)]),
               "has_wait": step_has_wait}
        cache.close()
        return res

    # GPU time of a step without refills (the initial map, one HIP graph of steps), to size the
    # visibility lag: the host loop itself paces the GPU, so its step time would overstate it
    m0 = np.full(E, -1, np.int32)
    m0[init] = np.arange(S, dtype=np.int32)
    map0 = torch.from_numpy(m0).cuda()
    n_cal = min(32, n_x)
    g_cal = capture(torch, comp, lambda t: B.moe_layer_forward(
        shape, xs[t], 1, wr, biases[t], map0, slots, ids_d[t], w_d[t], y_d[t], None, None, ws,
        stream=comp), n_cal)
    step_ms = time_graph(torch, B, comp, g_cal) / n_cal
    del g_cal
    lag = int(np.ceil(copy_ms / max(step_ms, 1e-3))) + 1
    log(f"calibration: refill batch {copy_ms:.3f} ms, GPU step {step_ms * 1e3:.1f} us -> lag {lag} steps")
    res = run(lag, n_x, True)
    st = res["stats"]
    sm = res["step_ms"][args.warmup:]
    hw = res["has_wait"][args.warmup:]
    base = float(np.median(sm[~hw])) if (~hw).any() else float(np.median(sm))
    stall_ms = float(np.sum(np.maximum(sm[hw] - base, 0.0))) if hw.any() else 0.0
    copy_total = float(np.sum(res["copy_ms"]))
    refill_bytes = st["refills"] * img
    gpu_ms = float(np.sum(sm))
    out = {
        "metric": "MoE-layer decode with an 8-slot expert cache: hit rate, hot-path tok/s, refill overlap",
        "value": round(steps / (gpu_ms / 1e3), 1), "unit": "tok/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "gptoss20b_8slots", "hidden": H, "inter": I, "n_experts": E, "top_k": k,
                   "slots": S, "policy": "LRU", "max_refills_per_step": 2, "lag_steps": lag,
                   "readback_delay_steps": 2, "drift_period": wl.drift_period},
        "hit_rate": round(st["hits"] / max(1, st["routes"]), 4),
        "refills": st["refills"], "evictions": st["evictions"],
        "refill_batch_ms_calibration": round(copy_ms, 4),
        "refill_gbs": round(refill_bytes / (copy_total * 1e-3) / 1e9, 2) if copy_total > 0 else None,
        "step_us_p50_p99": [round(float(np.percentile(sm, 50)) * 1e3, 2),
                            round(float(np.percentile(sm, 99)) * 1e3, 2)],
        "stall_us_total": round(stall_ms * 1e3, 1),
        "overlap": round(1.0 - stall_ms / copy_total, 4) if copy_total > 0 else None,
        "wall_tok_s": round(n_x / res["wall_s"], 1),
        "gpu_step_us_calibration": round(step_ms * 1e3, 2),
        "note": "host policy in a Python loop: the host paces the GPU (see slots8dev for the "
                "GPU-resident cache); GPU slots (105.75 MB) fit in the 256 MB Infinity Cache",
    }
    print(json.dumps(out), flush=True)
    return 0


# ---------------------------------------------------------------------------------------------
# stack48: 48 E=512 layers, half resident, residual chaining
# ---------------------------------------------------------------------------------------------
def bench_stack48(args):
    torch, B = setup()
    import synthetic
    from expert_offloaded_routed_amd import layer as L

    wl = synthetic.WORKLOADS["e512_verify_stack"]
    H, I, E, k, S, NL = wl.hidden, wl.inter, wl.n_experts, wl.top_k, wl.n_slots, wl.layers
    M = int(args.tokens)
    assert M in wl.tokens, f"--tokens must be one of {wl.tokens}"
    shape = B.make_shape(H, I, E, k, S)
    # a few generated layers' expert banks, byte-copied into every layer's own slots
    n_gen = 2
    t0 = time.time()
    banks = [L.pack_bank(shape, synthetic.experts_canonical(wl, l, range(E))) for l in range(n_gen)]
    log(f"generated {n_gen} layer banks in {time.time() - t0:.1f}s")
    img = banks[0].shape[1]
    wrs, biases, maps, slot_arrays = [], [], [], []
    # placement: each layer's own router (moe_route) over N_WARM warm-up tokens, one token per
    # step as in decode; experts ranked by route count (descending, then id), the top S resident
    N_WARM = 256
    ws_w = torch.zeros(B.moe_workspace_size(shape, N_WARM), dtype=torch.uint8, device="cuda")
    ids_w = torch.zeros((N_WARM, k), dtype=torch.int32, device="cuda")
    w_w = torch.zeros((N_WARM, k), dtype=torch.float32, device="cuda")
    for l in range(NL):
        wr_h = synthetic.router_weights(wl, l)
        bias_h = synthetic.zipf_bias(wl, l)
        xw = dev_bits(torch, np.concatenate([synthetic.activations(wl, 1, t, l, warmup=True)
                                             for t in range(N_WARM)]))
        wr_d, bias_d = dev_bits(torch, wr_h), torch.from_numpy(bias_h).cuda()
        B.moe_route(shape, xw, N_WARM, wr_d, bias_d, ids_w, w_w, ws_w)
        counts = np.bincount(ids_w.cpu().numpy().reshape(-1), minlength=E)
        order = sorted(range(E), key=lambda e: (-counts[e], e))[:S]
        slot_expert = np.array(order, np.int32)
        e2s = np.full(E, -1, np.int32)
        e2s[slot_expert] = np.arange(S, dtype=np.int32)
        wrs.append(wr_d)
        biases.append(bias_d)
        maps.append(torch.from_numpy(e2s).cuda())
        slot_arrays.append(L.device_slots(banks[l % n_gen], slot_expert, S))
    log(f"placed {NL} layers ({NL * S * img / 1e9:.1f} GB of slots)")
    args.steps = min(args.steps, 32)   # 48 layers x 4 launches per token step in one graph
    args.warmup = min(args.warmup, 4)
    n_tok = args.warmup + args.steps
    x0 = dev_bits(torch, np.concatenate([synthetic.activations(wl, M, t) for t in range(n_tok)]).reshape(n_tok, M, H))
    xa = torch.zeros((M, H), dtype=torch.int16, device="cuda")
    ws = torch.zeros(B.moe_workspace_size(shape, M), dtype=torch.uint8, device="cuda")
    ids_all = torch.zeros((args.steps, NL, M * k), dtype=torch.int32, device="cuda")
    cold_all = torch.zeros((args.steps, NL), dtype=torch.int32, device="cuda")
    w_d = torch.zeros((M, k), dtype=torch.float32, device="cuda")
    ids_d = torch.zeros((M, k), dtype=torch.int32, device="cuda")
    cold_d = torch.zeros((1,), dtype=torch.int32, device="cuda")
    cold_routes = torch.zeros((M * k,), dtype=torch.int32, device="cuda")
    y = torch.zeros((M, H), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()

    def token_step(t, rec=None):
        xa.copy_(x0[t])
        for l in range(NL):
            # the layer's kernels also form the next layer's input, bf16(x + y), in place
            B.moe_layer_forward_residual(shape, xa, M, wrs[l], biases[l], maps[l], slot_arrays[l],
                                         ids_d if rec is None else ids_all[rec, l].view(M, k), w_d,
                                         y, cold_d if rec is None else cold_all[rec, l:l + 1],
                                         cold_routes, xa, ws, stream=stream)

    with torch.cuda.stream(stream):
        for t in range(args.warmup):
            token_step(t)
    torch.cuda.synchronize()
    g = capture(torch, stream, lambda i: token_step(args.warmup + i, i), args.steps)
    torch.cuda.synchronize()
    ms = time_graph(torch, B, stream, g)
    ids_h = ids_all.cpu().numpy()
    cold_h = cold_all.cpu().numpy()
    hot_bytes = 0
    hits_layer = np.zeros(NL)
    maps_h = [m.cpu().numpy() for m in maps]
    exp_bytes = 3 * H * I // 2 + 3 * H * I // 32
    for s in range(args.steps):
        for l in range(NL):
            e = ids_h[s, l]
            hot = maps_h[l][e] >= 0
            hot_bytes += len(np.unique(e[hot])) * exp_bytes
            hits_layer[l] += hot.sum()
    assert np.array_equal(cold_h, np.array([[int((maps_h[l][ids_h[s, l]] < 0).sum()) for l in range(NL)]
                                            for s in range(args.steps)]))
    hit = hits_layer / (args.steps * M * k)
    tok_s = args.steps * M / (ms / 1e3)
    gbs = hot_bytes / (ms * 1e-3) / 1e9
    cpu = None
    if args.cpu_steps > 0:
        from oracle import layer as O
        NLB = 4  # layers of the sample
        cexp = [synthetic.experts_canonical(wl, l, range(E)) for l in range(n_gen)]
        routers = [(synthetic.router_weights(wl, l), synthetic.zipf_bias(wl, l)) for l in range(NLB)]

        def work(i):
            x = synthetic.activations(wl, M, i)
            for l in range(NLB):
                oid, ow, _, _ = O.route(O.router_logits(x, *routers[l]), k)
                y = O.layer_forward(x, oid, ow, cexp[l % n_gen], maps_h[l])["y_hot"]
                x = O.f64_to_bf16_rne(O.bf16_to_f64(x) + y)
        n_items = 24 if M == 1 else 8  # about 10 s of oracle work
        cpu = cpu_baseline(work, n_items, 2, M * NLB / NL, "tok/s",
                           f"token steps of {M} tokens through {NLB} of the {NL} layers (scaled to "
                           f"{NL}): float64 router, top-k, hot-only experts of each layer's placement, "
                           f"residual")
    out = {
        "metric": "48-layer E=512 MoE stack decode/verify tok/s, 256 of 512 experts resident per layer",
        "value": round(tok_s, 1), "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms / args.steps, 4), "higher_is_better": True,
        "dtype": "bf16", "data": f"synthetic; expert banks are byte copies of {n_gen} generated layers, "
                                 "routers, priors and placements are per layer",
        "config": {"workload": "e512_verify_stack", "hidden": H, "inter": I, "n_experts": E, "top_k": k,
                   "M": M, "layers": NL, "slots_per_layer": S,
                   "placement": f"warm-up popularity ({N_WARM} tokens routed by moe_route)",
                   "residual": "bf16(x + y) between layers", "timed": "one HIP graph of the token steps"},
        "hot_expert_gbs": round(gbs, 1), "frac_peak": round(gbs / PEAK_HBM_GBS, 4),
        "hot_bytes_per_token_step": int(hot_bytes / args.steps),
        "hit_rate_mean": round(float(hit.mean()), 4),
        "hit_rate_per_layer_min_max": [round(float(hit.min()), 4), round(float(hit.max()), 4)],
        "cold_routes_per_token_step": round(float(cold_h.sum()) / args.steps, 2),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


# ---------------------------------------------------------------------------------------------
# prefill: one E=512 layer, M=512, grouped GEMM
# ---------------------------------------------------------------------------------------------
def prefill_cpu_baseline(args, wl):
    """The oracle on whole prefill calls of the workload (router with its bias, top-k, every
    touched expert dequantised and multiplied in float64): the same output the GPU path forms."""
    import synthetic
    from oracle import layer as O
    M, k, E = wl.tokens[0], wl.top_k, wl.n_experts
    cexp = synthetic.experts_canonical(wl, 0, range(E))
    wr_h, bias_h = synthetic.router_weights(wl), synthetic.zipf_bias(wl)

    def work(i):
        x = synthetic.activations(wl, M, i)
        oid, ow, _, _ = O.route(O.router_logits(x, wr_h, bias_h), k)
        O.layer_forward(x, oid, ow, cexp)
    return cpu_baseline(work, 8, 1, M, "tok/s",
                        f"one call of {M} tokens: float64 router, top-k, dequantise-then-matmul of "
                        f"every touched expert")


def bench_prefill(args):
    torch, B = setup()
    import synthetic
    from expert_offloaded_routed_amd import layer as L

    wl = synthetic.WORKLOADS["e512_prefill"]
    H, I, E, k = wl.hidden, wl.inter, wl.n_experts, wl.top_k
    M = wl.tokens[0]
    shape = B.make_shape(H, I, E, k, E)
    t0 = time.time()
    bank = L.pack_bank(shape, synthetic.experts_canonical(wl, 0, range(E)))
    log(f"generated + packed {E} experts ({bank.nbytes / 1e6:.1f} MB) in {time.time() - t0:.1f}s")
    img = bank.shape[1]
    R = 4  # touched experts ~0.2 GB per call: 4 copies put the reuse distance beyond the MALL
    bd = torch.from_numpy(bank).cuda()
    copies = torch.empty((R, E, img), dtype=torch.uint8, device="cuda")
    for r in range(R):
        copies[r].copy_(bd)
    del bd
    wr = dev_bits(torch, synthetic.router_weights(wl))
    bias = torch.from_numpy(synthetic.zipf_bias(wl)).cuda()
    reps = max(4, min(args.steps, 32))
    xs = dev_bits(torch, np.stack([synthetic.activations(wl, M, t) for t in range(reps)]))
    ws = torch.zeros(B.moe_workspace_size(shape, M), dtype=torch.uint8, device="cuda")
    ids = torch.zeros((reps, M, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((reps, M, k), dtype=torch.float32, device="cuda")
    y = torch.zeros((M, H), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()

    def call(i):
        B.moe_layer_forward(shape, xs[i], M, wr, bias, None, copies[i % R], ids[i], w[i], y, None, None, ws,
                            stream=stream)

    with torch.cuda.stream(stream):
        for i in range(2):
            call(i)
    torch.cuda.synchronize()
    g = capture(torch, stream, call, reps)
    ms = time_graph(torch, B, stream, g) / reps
    ids_h = ids.cpu().numpy()
    exp_bytes = 3 * H * I // 2 + 3 * H * I // 32
    touched = np.mean([len(np.unique(ids_h[i])) for i in range(reps)])
    counts = np.bincount(ids_h[0].reshape(-1), minlength=E)
    flops = 2.0 * M * k * 3 * H * I
    gbs = touched * exp_bytes / (ms * 1e-3) / 1e9
    tfs = flops / (ms * 1e-3) / 1e12
    cpu = prefill_cpu_baseline(args, wl) if args.cpu_steps > 0 else None
    out = {
        "metric": "MoE-layer prefill (M=512) grouped GEMM: expert-weight GB/s and TFLOP/s",
        "value": round(M / (ms / 1e3), 1), "unit": "tok/s", "n_gpus": 1, "steps": reps, "warmup": 2,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "e512_prefill", "hidden": H, "inter": I, "n_experts": E, "top_k": k,
                   "M": M, "bank_copies": R, "timed": "one HIP graph of the calls"},
        "touched_experts_mean": round(float(touched), 1),
        "expert_gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        "tflops": round(tfs, 2), "frac_bf16_peak": round(tfs / PEAK_BF16_TFLOPS, 5),
        "routes_per_expert_max_mean": [int(counts.max()), round(float(counts[counts > 0].mean()), 2)],
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


# ---------------------------------------------------------------------------------------------
# slots8dev: 8 GPU slots, the GPU-resident cache, the whole decode loop in one HIP graph
# ---------------------------------------------------------------------------------------------
def _c3_setup(torch, B, L, synthetic, steps):
    wl = synthetic.WORKLOADS["gptoss20b_8slots"]
    H, I, E, k, S = wl.hidden, wl.inter, wl.n_experts, wl.top_k, wl.n_slots
    shape = B.make_shape(H, I, E, k, S)
    experts = synthetic.experts_canonical(wl, 0, range(E))
    bank_np = L.pack_bank(shape, experts)
    init = np.argsort(synthetic.zipf_ranks(wl))[:S].astype(np.int32)
    xs = dev_bits(torch, np.concatenate([synthetic.activations(wl, 1, t) for t in range(steps)]))
    biases = torch.from_numpy(np.stack([synthetic.zipf_bias(wl, 0, synthetic.drift_shift(wl, t))
                                        for t in range(steps)])).cuda()
    wr = dev_bits(torch, synthetic.router_weights(wl))
    return wl, shape, experts, bank_np, init, xs, biases, wr


def bench_slots8dev(args):
    torch, B = setup()
    import synthetic
    from expert_offloaded_routed_amd import layer as L

    steps = args.steps
    wl, shape, experts, bank_np, init, xs, biases, wr = _c3_setup(torch, B, L, synthetic, steps)
    H, E, k, S = wl.hidden, wl.n_experts, wl.top_k, wl.n_slots
    img = bank_np.shape[1]
    bank = L.pinned_bank(bank_np)
    slots = L.device_slots(bank_np, init, S)
    comp, copy = torch.cuda.Stream(), torch.cuda.Stream()
    ws = torch.zeros(B.moe_workspace_size(shape, 1), dtype=torch.uint8, device="cuda")
    ids = torch.full((steps, k), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((steps, k), dtype=torch.float32, device="cuda")
    y = torch.zeros((steps, H), dtype=torch.float32, device="cuda")
    maps = torch.zeros((steps, E), dtype=torch.int32, device="cuda")
    plans = torch.zeros((steps, 2 * B.REFILL_RECORD_BYTES), dtype=torch.uint8, device="cuda")
    nplan = torch.zeros((steps,), dtype=torch.int32, device="cuda")
    ev = [[B.event_create() for _ in range(steps)] for _ in range(3)]  # plan, layer, copy

    def build(cache, lag, refills, serial=False):
        # serial: the step's refills are copied on the compute stream right after the policy
        # kernel, before the layer
        def step(t):
            cache.step(ids[(t - 1) % steps], k, maps[t], plans[t], nplan[t:t + 1], stream=comp)
            B.event_record(ev[0][t], comp)
            if serial:
                cache.copy(nplan[t:t + 1], plans[t], bank, slots, stream=comp)
            elif refills and t - lag >= 0:
                B.stream_wait_event(comp, ev[2][t - lag])
            B.moe_layer_forward(shape, xs[t], 1, wr, biases[t], maps[t], slots, ids[t], w[t], y[t],
                                None, None, ws, stream=comp)
            B.event_record(ev[1][t], comp)
            if refills and not serial:
                B.stream_wait_event(copy, ev[0][t])
                if t >= 1:
                    B.stream_wait_event(copy, ev[1][t - 1])
                cache.copy(nplan[t:t + 1], plans[t], bank, slots, stream=copy)
                B.event_record(ev[2][t], copy)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(comp):
            with torch.cuda.graph(g, stream=comp):
                for t in range(steps):
                    step(t)
                if refills and not serial:
                    B.stream_wait_event(comp, ev[2][steps - 1])
        torch.cuda.synchronize()
        return g

    # calibration: GPU time of a step with no refills (static placement), and of the copy kernel
    # moving one refill batch (2 experts)
    cache0 = B.DeviceCache(shape, max_refills_per_step=0, initial_slot_expert=init, stream=comp)
    g0 = build(cache0, 1, False)
    t_hot = time_graph(torch, B, comp, g0) / steps
    calib = torch.zeros((2 * B.REFILL_RECORD_BYTES,), dtype=torch.uint8)
    rec = calib.numpy().view(np.int32).reshape(2, 6)
    rec[0, :4] = [init[0], 0, -1, 0]
    rec[1, :4] = [init[1], 1, -1, 0]
    plan_c, n_c = calib.cuda(), torch.tensor([2], dtype=torch.int32, device="cuda")
    e0, e1 = B.event_create(timing=True), B.event_create(timing=True)
    cache0.copy(n_c, plan_c, bank, slots, stream=copy)  # (untimed first launch)
    B.event_record(e0, copy)
    for _ in range(4):
        cache0.copy(n_c, plan_c, bank, slots, stream=copy)
    B.event_record(e1, copy)
    B.event_synchronize(e1)
    t_copy = B.event_elapsed_ms(e0, e1) / 4
    lag = int(np.ceil(t_copy / max(t_hot, 1e-6))) + 1
    log(f"calibration: step {t_hot * 1e3:.1f} us (GPU, no refills), copy kernel {t_copy:.3f} ms per "
        f"2 experts ({2 * img / (t_copy * 1e-3) / 1e9:.1f} GB/s) -> lag {lag} steps")

    # interference: the refill-free step graph replayed while the side stream runs (a) the copy
    # kernel over device-mapped host memory, (b) a DMA-engine copy from pinned host memory of the
    # same bytes; each side job is queued long enough to cover the whole replay
    def hot_step_beside(side):
        torch.cuda.synchronize()
        side()
        B.event_record(e0, comp)
        with torch.cuda.stream(comp):
            g0.replay()
        B.event_record(e1, comp)
        B.event_synchronize(e1)
        us = B.event_elapsed_ms(e0, e1) / steps * 1e3
        torch.cuda.synchronize()
        return us
    n_side = int(np.ceil(5.0 * steps * t_hot / t_copy)) + 1  # covers a replay slowed 5x
    dma_dst = torch.empty((2, img), dtype=torch.uint8, device="cuda")

    def copy_kernel_side():
        for _ in range(n_side):
            cache0.copy(n_c, plan_c, bank, slots, stream=copy)

    def dma_side():
        with torch.cuda.stream(copy):
            for _ in range(n_side):
                dma_dst.copy_(bank[:2], non_blocking=True)
    interference = {"hot_step_us_alone": round(t_hot * 1e3, 2),
                    "beside_copy_kernel": round(hot_step_beside(copy_kernel_side), 2),
                    "beside_dma_copy": round(hot_step_beside(dma_side), 2)}
    torch.cuda.synchronize()
    B.event_record(e0, copy)
    with torch.cuda.stream(copy):
        for _ in range(4):
            dma_dst.copy_(bank[:2], non_blocking=True)
    B.event_record(e1, copy)
    B.event_synchronize(e1)
    interference["dma_copy_gbs"] = round(4 * 2 * img / (B.event_elapsed_ms(e0, e1) * 1e-3) / 1e9, 2)
    del dma_dst, g0
    log(f"interference: {interference}")
    def run_mode(serial):
        # the same lag in both modes: it bounds the refill rate (at most 2 pending), so that both
        # move the same experts; in-stream the copies are simply done by then
        lag_m = lag
        slots.copy_(L.device_slots(bank_np, init, S))
        ids.fill_(-1)
        cache = B.DeviceCache(shape, lag_steps=lag_m, initial_slot_expert=init, stream=comp)
        g = build(cache, lag_m, True, serial)
        with torch.cuda.stream(comp):
            g.replay()  # warm-up replay (the cache state carries over to the timed one)
        torch.cuda.synchronize()
        s1 = cache.stats()
        t0, t1 = B.event_create(timing=True), B.event_create(timing=True)
        B.event_record(t0, comp)
        with torch.cuda.stream(comp):
            g.replay()
        B.event_record(t1, comp)
        B.event_synchronize(t1)
        ms = B.event_elapsed_ms(t0, t1)
        s2 = cache.stats()
        del g
        torch.cuda.synchronize()
        d = {f: s2[f] - s1[f] for f in s1}  # counters of the timed replay
        stall_ms = max(0.0, ms - steps * t_hot)
        copy_ms_total = d["refills"] / 2.0 * t_copy
        return {"tok_s": round(steps / (ms / 1e3), 1), "ms_per_step": round(ms / steps, 5),
                "lag_steps": lag_m, "hit_rate": round(d["hits"] / max(1, d["routes"]), 4),
                "refills": d["refills"], "stall_us_total": round(stall_ms * 1e3, 1),
                "overlap": (round(1.0 - stall_ms / copy_ms_total, 4) if copy_ms_total > 0 and not serial
                            else None)}

    side = run_mode(False)
    serial = run_mode(True)
    log(f"refills on a side stream: {side}; in the compute stream: {serial}")
    best = serial if serial["tok_s"] > side["tok_s"] else side
    best_serial = best is serial
    out = {
        "metric": "MoE-layer decode with an 8-slot GPU-resident expert cache: tok/s, hit rate, refill overlap",
        "value": best["tok_s"], "unit": "tok/s", "n_gpus": 1, "steps": steps,
        "warmup": steps, "ms_per_step": best["ms_per_step"], "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic (seeded MXFP4 experts, Zipf(1.1) prior drifting every 32 steps)",
        "config": {"workload": "gptoss20b_8slots_device_cache", "hidden": H, "inter": wl.inter,
                   "n_experts": E, "top_k": k, "slots": S, "policy": "LRU", "max_refills_per_step": 2,
                   "lag_steps": best["lag_steps"], "observes": "the previous step's routes, from device memory",
                   "refills": ("copy kernel in the compute stream, before the step's layer" if best_serial
                               else "copy kernel on a side stream"),
                   "timed": "one HIP graph of the steps: the policy kernel, then the layer in one "
                            "launch (router, route table, gate/up, down, combine), on the compute "
                            "stream"},
        "hit_rate": best["hit_rate"], "refills": best["refills"],
        "hot_step_us_no_refills": round(t_hot * 1e3, 2),
        "refill_batch_ms": round(t_copy, 4),
        "refill_gbs": round(2 * img / (t_copy * 1e-3) / 1e9, 2),
        "stall_us_total": best["stall_us_total"],
        "hot_step_us_beside_refill_copies": interference,
        "overlap_side_stream": side["overlap"],  # (in-stream copies do not overlap by design)
        "modes": {"side_stream": side, "in_stream": serial},
        "note": "GPU slots (105.75 MB) fit in the 256 MB Infinity Cache: hot-path bytes are cache-resident",
    }
    lag = best["lag_steps"]
    if args.cpu_steps > 0:
        from oracle import layer as O
        from oracle.cache_policy import SlotCachePolicy
        wr_h = synthetic.router_weights(wl)
        pol = SlotCachePolicy(E, S, init, max_refills=2, lag=lag, max_pending=2)
        prev = [None]

        def work(t):
            x = synthetic.activations(wl, 1, t)
            oid, ow, _, _ = O.route(O.router_logits(x, wr_h, synthetic.zipf_bias(
                wl, 0, synthetic.drift_shift(wl, t))), k)
            m, _ = pol.step(t, prev[0])
            prev[0] = oid
            O.layer_forward(x, oid, ow, experts, m)
        n = max(2, args.cpu_steps)
        out["cpu_baseline"] = cpu_baseline(work, n, max(1, n // 8), 1.0, "tok/s",
                                           "decode steps with the oracle's policy replay and the hot-only output")
    print(json.dumps(out), flush=True)
    return 0


# ---------------------------------------------------------------------------------------------
# hybrid: 8 GPU slots (static, the 8 most popular experts), cold routes on the host cores
# ---------------------------------------------------------------------------------------------
def bench_hybrid(args):
    torch, B = setup()
    import synthetic
    from expert_offloaded_routed_amd import layer as L

    steps = min(args.steps, 64)
    wl, shape, experts, bank_np, init, xs, biases, wr = _c3_setup(torch, B, L, synthetic, steps + 8)
    H, E, k, S = wl.hidden, wl.n_experts, wl.top_k, wl.n_slots
    bank = L.pinned_bank(bank_np)
    slots = L.device_slots(bank_np, init, S)
    e2s = np.full(E, -1, np.int32)
    e2s[init] = np.arange(S, dtype=np.int32)
    e2s_d = torch.from_numpy(e2s).cuda()
    buf = L.Buffers(shape, 1)
    st = B.HybridStaging(shape, 1)
    threads = nproc()
    stream = torch.cuda.Stream()
    ids_all = np.zeros((steps, k), np.int32)

    def call(t):
        B.moe_layer_forward_hybrid(shape, xs[t], 1, wr, biases[t], e2s_d, e2s, slots, bank.numpy(),
                                   buf.ids, buf.w, buf.y, st, buf.ws, n_threads=threads, stream=stream)

    for t in range(4):
        call(steps + t)
    torch.cuda.synchronize()
    tw = time.perf_counter()
    for t in range(steps):
        call(t)
        ids_all[t] = st.ids.numpy()[0]
    torch.cuda.synchronize()
    wall = time.perf_counter() - tw
    # the host part alone on the same routes, and the GPU part alone
    y_c = np.zeros((1, H), np.float32)
    th = time.perf_counter()
    for t in range(steps):
        B.moe_cold_forward_host(shape, bank.numpy(), xs[t:t + 1].cpu().numpy().view(np.uint16), 1,
                                ids_all[t:t + 1], np.full((1, k), 0.25, np.float32), e2s, y_c, threads)
    host_ms = (time.perf_counter() - th) / steps * 1e3
    cold = (e2s[ids_all] < 0).sum(axis=1)
    img = bank_np.shape[1]
    out = {
        "metric": "MoE-layer decode, hybrid: 8 hot experts on the GPU, cold routes on the host cores",
        "value": round(steps / wall, 2), "unit": "tok/s", "n_gpus": 1, "steps": steps, "warmup": 4,
        "ms_per_step": round(wall / steps * 1e3, 4), "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic", "config": {"workload": "gptoss20b_8slots_hybrid", "hidden": H,
                                        "inter": wl.inter, "n_experts": E, "top_k": k, "slots": S,
                                        "placement": "static: Zipf ranks 1..8", "host_threads": threads},
        "cold_routes_per_step": round(float(cold.mean()), 3),
        "host_cold_ms_per_step": round(host_ms, 3),
        "host_cold_gbs": round(float(cold.mean()) * img / (host_ms * 1e-3) / 1e9, 2) if host_ms > 0 else None,
        "note": "wall-clock per call: the host computes the cold routes while the GPU runs the hot ones",
        "cpu_baseline": None,
    }
    if args.cpu_steps > 0:
        from oracle import layer as O
        wr_h = synthetic.router_weights(wl)

        def work(t):
            x = synthetic.activations(wl, 1, t)
            oid, ow, _, _ = O.route(O.router_logits(x, wr_h, synthetic.zipf_bias(
                wl, 0, synthetic.drift_shift(wl, t))), k)
            O.layer_forward(x, oid, ow, experts)
        n = max(2, args.cpu_steps)
        out["cpu_baseline"] = cpu_baseline(work, n, max(1, n // 8), 1.0, "tok/s",
                                           "decode steps of the same layer, every route (the hybrid's "
                                           "full output): float64 router, top-k, dequantise-then-matmul")
    st.close()
    print(json.dumps(out), flush=True)
    return 0


# ---------------------------------------------------------------------------------------------
# staged: the E=512 prefill with every expert in host memory, 48 staging slots
# ---------------------------------------------------------------------------------------------
def bench_staged(args):
    torch, B = setup()
    import synthetic
    from expert_offloaded_routed_amd import layer as L

    wl = synthetic.WORKLOADS["e512_prefill"]
    H, I, E, k = wl.hidden, wl.inter, wl.n_experts, wl.top_k
    M = wl.tokens[0]
    n_slots = 48
    shape = B.make_shape(H, I, E, k, E)
    bank_np = L.pack_bank(shape, synthetic.experts_canonical(wl, 0, range(E)))
    bank = L.pinned_bank(bank_np)
    img = bank_np.shape[1]
    reps = max(3, min(args.steps, 8))
    xs = dev_bits(torch, np.stack([synthetic.activations(wl, M, t) for t in range(reps + 1)]))
    wr = dev_bits(torch, synthetic.router_weights(wl))
    bias = torch.from_numpy(synthetic.zipf_bias(wl)).cuda()
    st = B.PrefillStaging(shape, M, n_slots)
    buf = L.Buffers(shape, M)
    stream = torch.cuda.Stream()
    B.moe_layer_forward_staged(shape, xs[reps], M, wr, bias, bank, buf.ids, buf.w, buf.y, st, buf.ws,
                               stream=stream)
    torch.cuda.synchronize()
    tw = time.perf_counter()
    touched, passes = [], []
    for r in range(reps):
        nt, npass = B.moe_layer_forward_staged(shape, xs[r], M, wr, bias, bank, buf.ids, buf.w, buf.y,
                                               st, buf.ws, stream=stream)
        touched.append(nt)
        passes.append(npass)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - tw) / reps
    moved = float(np.mean(touched)) * img
    out = {
        "metric": "MoE-layer prefill (M=512) with staged experts: touched experts copied once from host memory",
        "value": round(M / wall, 1), "unit": "tok/s", "n_gpus": 1, "steps": reps, "warmup": 1,
        "ms_per_step": round(wall * 1e3, 4), "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "e512_prefill_staged", "hidden": H, "inter": I, "n_experts": E, "top_k": k,
                   "M": M, "staging_slots": n_slots, "resident": "none (every expert in pinned host memory)"},
        "touched_experts_mean": round(float(np.mean(touched)), 1), "passes": int(np.max(passes)),
        "staged_gbs": round(moved / wall / 1e9, 2),
        "note": "wall-clock per call; the host copies are PCIe-bound and overlap the passes' expert kernels",
        "cpu_baseline": prefill_cpu_baseline(args, wl) if args.cpu_steps > 0 else None,
    }
    st.close()
    print(json.dumps(out), flush=True)
    return 0


# ---------------------------------------------------------------------------------------------
# fate: next-layer routes predicted from the current layer's input (the next layer's router)
# ---------------------------------------------------------------------------------------------
def bench_fate(args):
    torch, B = setup()
    import synthetic
    from expert_offloaded_routed_amd import layer as L

    wl = synthetic.WORKLOADS["e512_verify_stack"]
    H, I, E, k = wl.hidden, wl.inter, wl.n_experts, wl.top_k
    NL, T = 8, min(args.steps, 64)
    shape = B.make_shape(H, I, E, k, E)
    slots = L.device_slots(L.pack_bank(shape, synthetic.experts_canonical(wl, 0, range(E))))
    wrs = [dev_bits(torch, synthetic.router_weights(wl, l)) for l in range(NL)]
    bs = [torch.from_numpy(synthetic.zipf_bias(wl, l)).cuda() for l in range(NL)]
    buf = L.Buffers(shape, 1)
    pred = L.Buffers(shape, 1)
    actual = np.zeros((T, NL, k), np.int32)
    predicted = np.zeros((T, NL, k), np.int32)
    x = torch.zeros((1, H), dtype=torch.int16, device="cuda")
    for t in range(T):
        x.copy_(dev_bits(torch, synthetic.activations(wl, 1, 9000 + t)))
        for l in range(NL):
            if l + 1 < NL:  # the next layer's router on this layer's input: the prediction
                B.moe_route(shape, x, 1, wrs[l + 1], bs[l + 1], pred.ids, pred.w, pred.ws)
                predicted[t, l + 1] = pred.ids[0].cpu().numpy()
            B.moe_layer_forward_residual(shape, x, 1, wrs[l], bs[l], None, slots, buf.ids, buf.w, buf.y,
                                         None, None, x, buf.ws)
            actual[t, l] = buf.ids[0].cpu().numpy()
    torch.cuda.synchronize()
    # recall of the prediction, and the hit rate of a small per-layer LRU set with and without
    # the predicted experts prefetched before the layer runs
    recall = np.mean([len(set(predicted[t, l]) & set(actual[t, l])) / k
                      for t in range(T) for l in range(1, NL)])
    S = 64
    hits = {"reactive": 0, "fate": 0}
    for mode in hits:
        for l in range(1, NL):
            lru = []  # most recent last
            for t in range(T):
                have = set(lru)
                if mode == "fate":
                    have |= set(predicted[t, l].tolist())
                hits[mode] += sum(1 for e in actual[t, l] if e in have)
                for e in (list(predicted[t, l]) if mode == "fate" else []) + list(actual[t, l]):
                    if e in lru:
                        lru.remove(e)
                    lru.append(int(e))
                lru = lru[-S:]
    n = T * (NL - 1) * k
    out = {
        "metric": "FATE next-layer prefetch: recall of the next layer's routes predicted from the current layer's input",
        "value": round(float(recall), 4), "unit": "fraction", "n_gpus": 1, "steps": T, "warmup": 0,
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "e512_stack_fate", "hidden": H, "inter": I, "n_experts": E, "top_k": k,
                   "layers": NL, "tokens": T, "lru_slots": S},
        "hit_rate_reactive_lru": round(hits["reactive"] / n, 4),
        "hit_rate_with_fate_prefetch": round(hits["fate"] / n, 4),
    }
    print(json.dumps(out), flush=True)
    return 0



# ---------------------------------------------------------------------------------------------
# formats: the decode workload with bf16, block FP8 or NVFP4 experts (the generic path)
# ---------------------------------------------------------------------------------------------
def _format_bytes(fmt, n, k):
    """Algorithmic bytes of one [n, k] matrix of the format: elements + scales."""
    el = {"bf16": 2 * n * k, "fp8_block": n * k, "nvfp4": n * k // 2}[fmt]
    sc = {"bf16": 0, "fp8_block": 4 * ((n + 127) // 128) * ((k + 127) // 128),
          "nvfp4": 4 + n * (k // 16)}[fmt]
    return el + sc


def bench_formats(args):
    torch, B = setup()
    import synthetic
    from expert_offloaded_routed_amd import layer as L

    wl = synthetic.WORKLOADS["gptoss20b_decode"]
    H, I, E, k = wl.hidden, wl.inter, wl.n_experts, wl.top_k
    fmt = args.format
    shape = B.make_shape(H, I, E, k, E, fmt)
    t0 = time.time()
    experts = synthetic.experts_canonical(wl, 0, range(E), fmt=fmt)
    bank = L.pack_bank(shape, experts)
    img = bank.shape[1]
    log(f"{fmt}: generated + packed {E} experts ({bank.nbytes / 1e6:.1f} MB) in {time.time() - t0:.1f}s")
    # copies of the bank at distinct addresses, at least 2 GB of them in all (no step finds its
    # experts in the Infinity Cache)
    R = max(2, min(args.copies, -(-2_000_000_000 // bank.nbytes)))
    bank_d = torch.from_numpy(bank).cuda()
    copies = torch.empty((R, E, img), dtype=torch.uint8, device="cuda")
    for r in range(R):
        copies[r].copy_(bank_d)
    del bank_d
    wr = dev_bits(torch, synthetic.router_weights(wl))
    bias = torch.from_numpy(synthetic.zipf_bias(wl)).cuda()
    n_x = args.warmup + args.steps
    xs = dev_bits(torch, np.concatenate([synthetic.activations(wl, 1, t) for t in range(n_x)]))
    ws = torch.zeros(B.moe_workspace_size(shape, 1), dtype=torch.uint8, device="cuda")
    ids = torch.zeros((n_x, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((n_x, k), dtype=torch.float32, device="cuda")
    y = torch.zeros((n_x, H), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()

    def step(t):
        B.moe_layer_forward(shape, xs[t], 1, wr, bias, None, copies[t % R], ids[t], w[t], y[t], None,
                            None, ws, stream=stream)

    with torch.cuda.stream(stream):
        for t in range(args.warmup):
            step(t)
    torch.cuda.synchronize()
    g_timed = capture(torch, stream, lambda i: step(args.warmup + i), args.steps)
    torch.cuda.synchronize()
    ms_total = time_graph(torch, B, stream, g_timed)
    ms_step = ms_total / args.steps
    ids_h = ids[args.warmup:].cpu().numpy()
    srt = np.sort(ids_h, axis=1)
    assert np.all(srt[:, 1:] != srt[:, :-1])
    assert np.isfinite(y[args.warmup:].cpu().numpy()).all()
    gu_bytes = k * 2 * _format_bytes(fmt, I, H)
    dn_bytes = k * _format_bytes(fmt, H, I)
    step_bytes = gu_bytes + dn_bytes

    # stage timing with the marked calls, back to back behind a spin kernel (as for decode)
    n_st = max(1, min(args.stage_steps, args.steps))
    marks = [[B.event_create(timing=True, system_fence=False) for _ in range(4)] for _ in range(n_st)]
    for rep in range(2):
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            torch.cuda._sleep(int(args.enqueue_spin_cycles))
            for i in range(n_st):
                t = args.warmup + i
                B.moe_layer_forward_marked(shape, xs[t], 1, wr, bias, None, copies[t % R], ids[t], w[t],
                                           y[t], None, None, ws, marks[i], stream=stream)
    torch.cuda.synchronize()
    st = np.array([[B.event_elapsed_ms(m[j], m[j + 1]) for j in range(3)] for m in marks]) * 1e3
    for m in marks:
        for e in m:
            B.event_destroy(e)
    us_rt, us_gu, us_dn = (float(v) for v in st.mean(axis=0))
    gu_gbs = gu_bytes / (us_gu * 1e-6) / 1e9
    dn_gbs = dn_bytes / (us_dn * 1e-6) / 1e9
    ceil_gbs, ceil_us = stream_ceiling(torch, B, copies.view(-1), gu_bytes, stream)
    log(f"{fmt}: read-streaming ceiling {ceil_gbs:.0f} GB/s ({ceil_us:.2f} us per {gu_bytes} B)")

    cpu = None
    if args.cpu_steps > 0:
        from oracle import layer as O
        wr_h = synthetic.router_weights(wl)
        bias_h = synthetic.zipf_bias(wl)
        def work(t):
            x = synthetic.activations(wl, 1, t)
            oid, ow, _, _ = O.route(O.router_logits(x, wr_h, bias_h), k)
            O.layer_forward(x, oid, ow, experts)
        n_cpu = max(1, args.cpu_steps // 4)
        cpu = cpu_baseline(work, n_cpu, max(1, n_cpu // 4), 1.0, "tok/s",
                           f"decode steps (M=1) of the same layer: float64 router, top-k and "
                           f"dequantise-then-matmul of the 4 routed {fmt} experts")

    out = {
        "metric": f"MoE-layer decode tok/s at M=1, {fmt} experts (generic path) + achieved HBM GB/s",
        "value": round(args.steps / (ms_total / 1e3), 1), "unit": "tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": f"synthetic (seeded N(0,0.02) weights -> {fmt}, N(0,1) bf16 activations, Zipf(1.1) prior)",
        "config": {"workload": f"gptoss20b_decode_{fmt}", "hidden": H, "inter": I, "n_experts": E,
                   "top_k": k, "M": 1, "format": fmt, "resident": "all", "bank_copies": R,
                   "timed": "one HIP graph of the steps"},
        "expert_bytes_per_step": step_bytes,
        "hbm_gbs_step": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "stage_us": {"route (router GEMV + top-k / bucketing)": round(us_rt, 2),
                     "gateup (generic gate/up + SiLU*up)": round(us_gu, 2),
                     "down (generic down + ordered combine)": round(us_dn, 2)},
        "down_gbs": round(dn_gbs, 1),
        "roofline": {"bound": "hbm", "kernel": f"k_gateup_fmt<{fmt}> (gate/up GEMV + SiLU*up)",
                     "achieved": round(gu_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "bytes_per_launch": gu_bytes, "us_per_launch": round(us_gu, 3),
                     "launches_timed": n_st, "measured_ceiling_gbs": round(ceil_gbs, 1),
                     "frac_of_measured_ceiling": round(gu_gbs / ceil_gbs, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def write_traffic(fetch_csv, write_csv):
    """profiles/traffic.json from the counter CSVs of the two passes over the decode line: the
    median FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the fused decode kernel and of the
    streaming probe, each scaled by what the same counter reads for the plain device copy of
    --calibrate-copy-mb (the last four copy dispatches), keyed by the kernel sources' hash."""
    import csv
    from expert_offloaded_routed_amd import _build

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")

    def pick(vals, prefix):
        rows = [v for k, v in vals.items() if prefix in k]
        if len(rows) != 1:
            raise SystemExit(f"expected one kernel matching {prefix!r}, found {len(rows)}")
        return rows[0]
    copy_f = pick(fetch, "copyBuffer")[-4:]
    copy_w = pick(write, "copyBuffer")[-4:]
    nbytes = 256 << 20
    fs = nbytes / (float(np.median(copy_f)) * 1024)
    ws = nbytes / (float(np.median(copy_w)) * 1024)
    out = {"kernel_source_sha": _build.kernel_source_sha(),
           "copy_calibration": {"bytes": nbytes, "fetch_size_kib": float(np.median(copy_f)),
                                "write_size_kib": float(np.median(copy_w)),
                                "fetch_scale": round(fs, 6), "write_scale": round(ws, 6)}}
    algo = {"layer_decode": 52876800, "stream_probe": 52876800}
    for name, prefix in (("layer_decode", "k_layer_decode"), ("stream_probe", "k_stream_probe")):
        f, w = pick(fetch, prefix), pick(write, prefix)
        fm, wm = float(np.median(f)), float(np.median(w))
        hbm = int(round(fm * 1024 * fs + wm * 1024 * ws))
        out[name] = {"fetch_size_kib_median": fm, "write_size_kib_median": wm,
                     "dispatches": [len(f), len(w)], "hbm_bytes_per_launch": hbm,
                     "algorithmic_bytes_per_launch": algo[name],
                     "ratio": round(hbm / algo[name], 4)}
    out["layer_decode_bytes_per_launch"] = out["layer_decode"]["hbm_bytes_per_launch"]
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out), flush=True)
    return 0


def copy_calibration(mib):
    """A plain device-to-device copy of known size (4 times): its HBM byte counters per launch
    give the scale between what the counters read and the bytes moved."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: 4 x {n} bytes device to device")


def main():
    args = parse()
    if args.traffic:
        return write_traffic(*args.traffic)
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1", "n_gpus": args.gpus}))
        return 2
    rc = {"decode": bench_decode, "slots8": bench_slots8, "slots8dev": bench_slots8dev,
          "hybrid": bench_hybrid, "stack48": bench_stack48, "prefill": bench_prefill,
          "staged": bench_staged, "fate": bench_fate, "formats": bench_formats}[args.workload](args)
    if args.calibrate_copy_mb > 0:
        copy_calibration(args.calibrate_copy_mb)
    return rc


if __name__ == "__main__":
    sys.exit(main())
