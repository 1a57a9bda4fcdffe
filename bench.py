"""Benchmark: grouped routed-expert MoE decode on one MI355X.

Workload (seeded, synthetic, shaped like the pages' measurements): 48 MoE layers, each with its own
128 experts in a 4-bit nonlinear format (NL4: 32 weights per 18-byte block), n_embd 2560, n_ff 768,
top-8 routing of one token (T = 1). All 48 x 128 experts are resident (20.4 GB pool), so each
pass reads its routed experts cold (1.27 GB per pass, far above the 256 MB Infinity Cache).

A step is one pass of the whole path over the 48 layers: top-k routing of the layer's logits,
grouping of the entries by expert, and the single-launch layer decode (q8_1 of x, grouped gate/up,
SwiGLU + q8_1, grouped down, weighted scatter). Steps are replayed from a HIP graph.

Printed: one JSON line. value = expert-weight GB/s (distinct routed experts' bytes per pass / time
per pass); us_per_layer_call = time per layer; roofline = the layer-decode kernel alone, timed
with HIP events around each launch; cpu_baseline = the CPU oracle on a sample of layers.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_graph(graph, n):
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(n):
        graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / n, (time.perf_counter() - t0) * 1e3 / n


def decode_kernel_us(wl, reps):
    """Average duration of the layer-decode launch, HIP events around each launch on its stream."""
    import torch
    s = torch.cuda.current_stream()
    evs = []
    for _ in range(reps):
        for l in range(wl.L):
            wl.route_plan(l)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(s)
            wl.decode(l)
            b.record(s)
            evs.append((a, b))
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    return sum(ts) / len(ts), ts[len(ts) // 2]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="nl4_2560x768_t1")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle time to measure")
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard by expert groups; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from moe_routed_expert_route_amd import binding as B
    from moe_routed_expert_route_amd.workloads import Workload

    B.lib()
    torch.cuda.set_device(0)
    log("building workload")
    wl = Workload(args.workload, device="cuda", log=log)
    per_layer = wl.weight_bytes_per_layer()
    bytes_pass = float(sum(per_layer))
    log(f"pool {wl.pool_bytes / 1e9:.2f} GB, routed bytes per pass {bytes_pass / 1e9:.3f} GB")

    # eager warm-up (also checks the plans)
    wl.step()
    torch.cuda.synchronize()
    errs = [p.errors() for p in wl.plans]
    assert not any(errs), errs

    # graph of one step (48 x [route, plan, decode])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        wl.step()
    torch.cuda.synchronize()
    # decode-only graph (48 x decode), plans already built
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, stream=s):
        for l in range(wl.L):
            wl.decode(l)
    torch.cuda.synchronize()

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    ms_step, wall_ms = time_graph(g, args.steps)
    ms_dec, _ = time_graph(g2, args.steps)
    # plain stream, no graph
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        wl.step()
    torch.cuda.synchronize()
    ms_plain = (time.perf_counter() - t0) * 1e3 / 3
    log("per-launch kernel timing")
    k_avg_us, k_med_us = decode_kernel_us(wl, 2)

    us_layer = ms_step * 1e3 / wl.L
    gbs = bytes_pass / (ms_step * 1e-3) / 1e9
    bytes_layer = bytes_pass / wl.L
    achieved = bytes_layer / (k_avg_us * 1e-6) / 1e9
    res = {
        "metric": "us per MoE-layer decode call at T=1..4; expert-weight GB/s (frac of HBM peak)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 dot (v_dot4) with fp32 scales",
        "data": "synthetic (seeded), random-init experts",
        "config": {"workload": f"{wl.L} layers x {wl.E} experts {args.workload}: n_embd {wl.n_embd}, "
                               f"n_ff {wl.n_ff}, top-{wl.k}, T={wl.T}, cold pool "
                               f"{wl.pool_bytes / 1e9:.1f} GB",
                   "layers": wl.L, "experts": wl.E, "n_embd": wl.n_embd, "n_ff": wl.n_ff,
                   "top_k": wl.k, "T": wl.T, "parallelism": "single GPU"},
        "us_per_layer_call": round(us_layer, 3),
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "us_per_layer_decode_only": round(ms_dec * 1e3 / wl.L, 3),
        "us_per_layer_plain_stream": round(ms_plain * 1e3 / wl.L, 3),
        "roofline": {"bound": "hbm", "kernel": "moe_layer_decode (k_layer)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": int(bytes_layer), "avg_launch_us": round(k_avg_us, 3),
                     "median_launch_us": round(k_med_us, 3)},
    }
    if not args.no_cpu:
        res["cpu_baseline"] = run_cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def run_cpu_baseline(wl, seconds):
    """The CPU oracle, as it stands, on the same workload: whole layer calls (route, group,
    quantize, gate/up, SwiGLU, q8_1, down, scatter), cycling over the layers until about
    `seconds` of oracle time have been measured. Weight generation is outside the timed part."""
    import numpy as np

    import oracle
    tb = oracle.Tables(wl.tables["nl4"], wl.tables["cb2"], wl.tables["cb3"])
    log(f"cpu oracle for ~{seconds} s")
    cache = {}
    total, calls, l = 0.0, 0, 0
    while total < seconds and calls < 4 * wl.L:
        if l not in cache:
            ids, w = oracle.route_topk(wl.logits[l], wl.k)
            ex = {int(e): wl.host_expert(l, int(e)) for e in np.unique(ids)}
            cache[l] = ex
        ex = cache[l]
        t0 = time.perf_counter()
        ids, w = oracle.route_topk(wl.logits[l], wl.k)
        plan = oracle.build_plan(ids, w.astype(np.float32), None, wl.E, 0)
        oracle.layer(wl.x[l], plan, wl.fg, wl.fd, {e: v[0] for e, v in ex.items()},
                     {e: v[1] for e, v in ex.items()}, {e: v[2] for e, v in ex.items()},
                     wl.n_embd, wl.n_ff, np.zeros((wl.T, wl.n_embd), np.float32), tb)
        total += time.perf_counter() - t0
        calls += 1
        l = (l + 1) % wl.L
    us = total / calls * 1e6
    return {"value": round(us, 1), "unit": "us per layer call", "cores": 1, "kind": "oracle",
            "sample": f"{calls} layer calls cycling over the {wl.L} layers of the same workload "
                      f"(same weights, logits and x); single-threaded plain-C oracle, float64 "
                      f"sums; {total:.1f} s measured, weight generation excluded",
            "gbs": round(sum(wl.weight_bytes_per_layer()) / wl.L * calls / total / 1e9, 3)}


if __name__ == "__main__":
    main()
