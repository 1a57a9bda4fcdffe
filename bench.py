"""Benchmark: grouped routed-expert MoE decode on one MI355X.

Headline workload (seeded, synthetic, shaped like the pages' measurements): 48 MoE layers, each
with its own 128 experts in the 4-bit nonlinear format (NL4: 32 weights per 18-byte block),
n_embd 2560, n_ff 768, top-8 routing of one token (T = 1). All 48 x 128 experts are resident
(20.4 GB pool), so a pass reads its routed experts cold (1.27 GB per pass, far above the 256 MB
last-level cache).

A step is one pass of the whole path over the 48 layers, two launches per layer: (1) top-k
routing of the layer's logits, grouping of the entries by expert, q8_1 of x, grouped gate/up,
SwiGLU + q8_1 of h; (2) grouped down + weighted scatter into Y. Steps are replayed from a HIP
graph.

Printed: one JSON line. value = expert-weight GB/s (distinct routed experts' bytes per pass / the
median time per pass over the timed replays, each replay bracketed by its own HIP events);
us_per_layer_call = time per layer; roofline = the dominant kernel alone (a HIP graph of its 48
launches, the median of several replays between HIP events on its stream), with the committed
rocprofv3 trace's figure beside it when the kernel sources are the traced ones; in-line
comparisons (planar vs row-major, one vs two calls) alternate their arms A B / B A; t_sweep = the
same measurement at T = 1..4 (shared experts: the per-extra-row cost; the 256-expert CB3/Q8_0
geometry with uniform routing); cpu_baseline = the CPU oracle on a sample of layer calls, on one
thread and on all cores.
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


def source_digest():
    """SHA-256 of what the kernels' machine code follows from: the sources and the build flags."""
    from moe_routed_expert_route_amd.profsum import source_digest as d
    return d()


def barrier():
    import torch.distributed as dist
    if dist.is_available() and dist.is_initialized():
        dist.barrier()


def replay_ms(graph, n, stream=None):
    """ms of each of n replays of `graph` (a HIP event after every replay, on the stream the
    replays run on), bracketed by a barrier and a device synchronize on both sides."""
    import torch
    barrier()
    torch.cuda.synchronize()
    st = stream if stream is not None else torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    with torch.cuda.stream(st):
        ev[0].record(st)
        for i in range(n):
            graph.replay()
            ev[i + 1].record(st)
    torch.cuda.synchronize()
    barrier()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]


def median(v):
    import numpy as np
    return float(np.median(np.asarray(v, dtype=np.float64)))


def time_graph(graph, n):
    """Median ms per replay of `graph` over n replays."""
    return median(replay_ms(graph, n))


def alternate(graphs, rounds=6, per=5):
    """In-line A/B comparison: the graphs (name -> graph) replayed in turn, A B, B A, A B, ... for
    `rounds` rounds of `per` replays each (so a clock change of the card falls on both arms), every
    replay timed with its own HIP events. Returns name -> {median ms, per-visit medians}."""
    names = list(graphs)
    times = {k: [] for k in names}
    visits = {k: [] for k in names}
    for r in range(rounds):
        for k in (names if r % 2 == 0 else names[::-1]):
            t = replay_ms(graphs[k], per)
            times[k] += t
            visits[k].append(round(median(t), 4))
    return {k: {"median_ms": median(times[k]), "visit_medians_ms": visits[k],
                "replays": len(times[k])} for k in names}


def kernel_us(wl, reps):
    """Duration of each launch kind (gate/up, down): a HIP graph of the kind's launches for every
    layer, each of `reps` replays timed between HIP events on its stream; the median replay divided
    by the launch count (kernels of one graph run back to back, so this is the kernels' own time)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    out = {}
    for kind, fn in (("gate_up", wl.gate_up), ("down", wl.down)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for l in range(wl.L):
                fn(l)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        out[kind] = median(replay_ms(g, reps, stream=s)) * 1e3 / wl.L
        del g
    return out


def measure(wl, steps, warmup, reps=9):
    """Graph-replayed step time (median of `steps` replays), plain-stream step time and per-kernel
    launch times."""
    import torch
    wl.step()
    torch.cuda.synchronize()
    errs = [p.errors() for p in wl.plans]
    assert not any(errs), errs
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        wl.step()
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    per = replay_ms(g, steps)
    ms_step = median(per)
    wl.last_replays = per
    t0 = time.perf_counter()
    for _ in range(3):
        wl.step()
    torch.cuda.synchronize()
    ms_plain = (time.perf_counter() - t0) * 1e3 / 3
    ks = kernel_us(wl, reps)
    del g
    return ms_step, ms_plain, ks


def step_graph(wl):
    """A HIP graph of one step of the workload (captured on a side stream), replayed once."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        wl.step()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    return g


def stream_read_gbs(gib=2, reps=7):
    """The library's own streaming read (moe_stream_read: 16-byte non-temporal loads, eight in
    flight per lane, every CU an equal share) over `gib` GiB, for a few grid sizes; each launch
    timed with HIP events on its stream, the median of `reps` per grid, the best grid reported:
    the bandwidth a plain read reaches from HBM on this device, beside the 8 TB/s peak."""
    import numpy as np
    import torch

    from moe_routed_expert_route_amd import binding as B
    n = gib << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.view(torch.int32).copy_(torch.arange(n // 4, dtype=torch.int32, device="cuda"))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(64 * cus, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    res = {}
    with torch.cuda.stream(s):
        for m in (4, 8, 16, 32, 64):
            grid = m * cus
            B.moe_stream_read(buf, out, grid, stream=s)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            ev[0].record(s)
            for i in range(reps):
                B.moe_stream_read(buf, out, grid, stream=s)
                ev[i + 1].record(s)
            torch.cuda.synchronize()
            res[grid] = median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])
    # the XOR of the workgroups' words is the buffer's: words 0..n/4-1, so x ^ (x + 1) pairs cancel
    got = int(np.bitwise_xor.reduce(out[:grid].cpu().numpy().astype(np.uint32)))
    assert got == 0, f"stream read checksum {got:#x}"
    best = min(res, key=res.get)
    del buf
    torch.cuda.empty_cache()
    return {"gbs": round(n / (res[best] * 1e-3) / 1e9, 1), "bytes": n, "grid": best,
            "workgroup_threads": 256,
            "gbs_by_grid": {str(g): round(n / (t * 1e-3) / 1e9, 1) for g, t in res.items()},
            "kind": "moe_stream_read (this library's k_stream_read: 16-byte non-temporal loads, "
                    "8 per lane in flight, every CU an equal share), HIP events, median of 7 "
                    "launches per grid, best grid"}


def empty_call_us(layers=48, reps=20):
    """Cost of a call with no work (n_groups = 0) at the 4096 x 1536 Q8_0 edge geometry, 256
    experts, plan capacity 32 entries from entry 7: a HIP graph of `layers` fused calls
    (moe_layer_decode), timed with HIP events."""
    import torch

    from moe_routed_expert_route_amd import binding as B
    from moe_routed_expert_route_amd import synth
    n_embd, n_ff, E = 4096, 1536, 256
    d = torch.device("cuda")
    zg = torch.zeros(synth.row_bytes(synth.Q8_0, n_embd) * n_ff, dtype=torch.uint8, device=d)
    zd = torch.zeros(synth.row_bytes(synth.Q8_0, n_ff) * n_embd, dtype=torch.uint8, device=d)
    t64 = dict(dtype=torch.int64, device=d)
    layer = B.Layer.from_pointers(n_embd, n_ff, synth.Q8_0, synth.Q8_0,
                                  torch.full((E,), zg.data_ptr(), **t64), torch.full((E,), zg.data_ptr(), **t64),
                                  torch.full((E,), zd.data_ptr(), **t64), keep=(zg, zd))
    plan = B.Plan(32, 32, entry_capacity=7 + 32, device=d)
    plan.set(synth.direct_plan(0, E, 4, 64, 7, 5, max_entries=32))
    x = torch.zeros((4, n_embd), dtype=torch.float32, device=d)
    Y = torch.zeros((64, n_embd), dtype=torch.float32, device=d)
    ws = B.workspace(layer, plan)
    B.moe_layer_decode(layer, plan, x, Y, ws)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(layers):
            B.moe_layer_decode(layer, plan, x, Y, ws)
    torch.cuda.synchronize()
    g.replay()
    ms = time_graph(g, reps)
    assert plan.errors() == 0
    del g
    return {"us_per_call": round(ms * 1e3 / layers, 3), "calls": layers,
            "config": "4096 x 1536 Q8_0, 256 experts, n_groups 0, cap 32 entries from entry 7, two launches"}


def two_calls_us(wl, reps=20):
    """Each layer as two fused calls (moe_layer_decode) sharing the entry arrays and Y: the routed
    plan of the layer split so that the groups of its two highest expert ids go to the second call
    (entries past the first call's), against one fused call with the whole plan. HIP graphs of the
    48 (or 96) calls, timed with HIP events."""
    import torch

    from moe_routed_expert_route_amd import binding as B
    from moe_routed_expert_route_amd import synth
    cap = wl.T * wl.k
    d = torch.device("cuda")
    one, first, second = [], [], []
    n2 = []
    for l in range(wl.L):
        ph = wl.plans[l].get()
        late = set(int(e) for e in ph["grp_expert"][-2:])
        pa, pb = synth.split_plan(ph, lambda e: e not in late)
        p1 = B.Plan(cap, cap, device=d)
        p1.set(ph)
        pa_d = B.Plan(cap, cap, device=d)
        pb_d = B.Plan(cap, cap, device=d, entries_of=pa_d)
        pa_d.set(pa)
        pb_d.set(pb)
        one.append(p1)
        first.append(pa_d)
        second.append(pb_d)
        n2.append(pb["n_groups"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graphs = {}
    for name, calls in (("one_call", [(one[l],) for l in range(wl.L)]),
                        ("two_calls", [(first[l], second[l]) for l in range(wl.L)])):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for l in range(wl.L):
                for p in calls[l]:
                    B.moe_layer_decode(wl.layers[l], p, wl.d_x[l], wl.Y[l], wl.ws[l])
        torch.cuda.synchronize()
        g.replay()
        graphs[name] = g
    ab = alternate(graphs, rounds=6, per=max(2, reps // 4))
    out = {k: v["median_ms"] * 1e3 / wl.L for k, v in ab.items()}
    del graphs
    assert not any(p.errors() for p in one + first)
    return {"us_per_layer_one_call": round(out["one_call"], 3),
            "us_per_layer_two_calls": round(out["two_calls"], 3),
            "us_second_call": round(out["two_calls"] - out["one_call"], 3),
            "groups_in_second_call": sorted(set(n2)),
            "ab": {k: v["visit_medians_ms"] for k, v in ab.items()},
            "config": "plan given (routed once beforehand), moe_layer_decode per call, graph of all "
                      "layers; the two graphs alternated A B / B A over 6 rounds, medians"}


def prefill_line(T=512, layers=2, reps=10):
    """The prompt path at T tokens on the headline geometry (NL4 2560 x 768, 128 experts, top-8):
    per layer quantize, route, plan, gate/up and down on the matrix cores, SwiGLU + q8_1, scatter,
    each layer's 128 experts in its own pool (every expert is routed at this T, so a layer reads
    all 128 experts' 425 MB once). HIP graphs of `layers` layers; per-kernel graphs of the two
    GEMM launches alone."""
    import numpy as np
    import torch

    from moe_routed_expert_route_amd import binding as B
    from moe_routed_expert_route_amd import synth
    n_embd, n_ff, E, k, fmt = 2560, 768, 128, 8, synth.NL4
    d = torch.device("cuda")
    sz_g, sz_d = synth.row_bytes(fmt, n_embd) * n_ff, synth.row_bytes(fmt, n_ff) * n_embd
    distinct = 16   # drawn experts, tiled over the 128 slots of each pool
    base_g = [torch.from_numpy(synth.weight_matrix(fmt, n_ff, n_embd, 90, e, 0)).to(d) for e in range(distinct)]
    base_u = [torch.from_numpy(synth.weight_matrix(fmt, n_ff, n_embd, 90, e, 1)).to(d) for e in range(distinct)]
    base_d = [torch.from_numpy(synth.weight_matrix(fmt, n_embd, n_ff, 90, e, 2)).to(d) for e in range(distinct)]
    nl4 = torch.from_numpy(synth.nl4_table(90)).to(d)
    L = []
    for l in range(layers):
        pg = torch.empty(E * sz_g, dtype=torch.uint8, device=d)
        pu = torch.empty(E * sz_g, dtype=torch.uint8, device=d)
        pd = torch.empty(E * sz_d, dtype=torch.uint8, device=d)
        for e in range(E):
            pg[e * sz_g:(e + 1) * sz_g].copy_(base_g[(e + l) % distinct])
            pu[e * sz_g:(e + 1) * sz_g].copy_(base_u[(e + l) % distinct])
            pd[e * sz_d:(e + 1) * sz_d].copy_(base_d[(e + l) % distinct])
        i64 = dict(dtype=torch.int64, device=d)
        lay = B.Layer.from_pointers(n_embd, n_ff, fmt, fmt,
                                    torch.tensor([pg.data_ptr() + e * sz_g for e in range(E)], **i64),
                                    torch.tensor([pu.data_ptr() + e * sz_g for e in range(E)], **i64),
                                    torch.tensor([pd.data_ptr() + e * sz_d for e in range(E)], **i64),
                                    nl4=nl4, keep=(pg, pu, pd))
        n = T * k
        st = dict(lay=lay, plan=B.Plan(E, n, device=d),
                  logits=torch.from_numpy(synth.router_logits(T, E, 91, l)).to(d),
                  x=torch.from_numpy(synth.activations(T, n_embd, 92, l)).to(d),
                  ids=torch.empty((T, k), dtype=torch.int32, device=d),
                  w=torch.empty((T, k), dtype=torch.float32, device=d),
                  ent_of=torch.empty((T, k), dtype=torch.int32, device=d),
                  xq=torch.empty((T, n_embd // 32 * 36), dtype=torch.uint8, device=d),
                  g=torch.empty((n, n_ff), dtype=torch.float32, device=d),
                  u=torch.empty((n, n_ff), dtype=torch.float32, device=d),
                  hq=torch.empty((n, n_ff // 32 * 36), dtype=torch.uint8, device=d),
                  O=torch.empty((n, n_embd), dtype=torch.float32, device=d),
                  Y=torch.zeros((T, n_embd), dtype=torch.float32, device=d))
        L.append(st)
    del base_g, base_u, base_d

    def layer(st, part="all"):
        if part in ("all", "pre"):
            B.moe_quantize_q8_1(st["x"], q=st["xq"])
            B.moe_route_topk(st["logits"], k, ids=st["ids"], w=st["w"])
            B.moe_prefill_plan(st["ids"], st["w"], st["plan"], E, ent_of=st["ent_of"])
        if part in ("all", "gate_up"):
            B.moe_prefill_gate_up(st["lay"], st["plan"], st["xq"], st["g"], st["u"])
        if part == "all":
            B.moe_prefill_swiglu_q8_1(st["plan"], st["g"], st["u"], n_ff, st["hq"])
        if part in ("all", "down"):
            B.moe_prefill_down(st["lay"], st["plan"], st["hq"], st["O"])
        if part == "all":
            B.moe_prefill_scatter(st["plan"], st["ent_of"], st["O"], st["Y"], n_embd)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    out = {}
    for part in ("all", "gate_up", "down"):
        for st in L:   # a full pass first, so the per-kernel graphs run on real plans
            layer(st)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for st in L:
                layer(st, part)
        torch.cuda.synchronize()
        g.replay()
        out[part] = time_graph(g, reps) * 1e3 / layers
        del g
    assert not any(st["plan"].errors() for st in L)
    ng = [int(st["plan"].n_groups.item()) for st in L]
    wbytes = float(np.mean(ng)) * (2 * sz_g + sz_d)
    macs = T * k * 3 * n_ff * n_embd
    res = {"T": T, "layers": layers, "experts_touched_per_layer": float(np.mean(ng)),
           "us_per_layer": round(out["all"], 2), "gate_up_us": round(out["gate_up"], 2),
           "down_us": round(out["down"], 2),
           "weight_gbs": round(wbytes / (out["all"] * 1e-6) / 1e9, 1),
           "int8_tops": round(2 * macs / (out["all"] * 1e-6) / 1e12, 2)}
    gu_bytes = float(np.mean(ng)) * 2 * sz_g
    res["roofline_gate_up"] = {"bound": "hbm", "achieved": round(gu_bytes / (out["gate_up"] * 1e-6) / 1e9, 1),
                               "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(gu_bytes / (out["gate_up"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                               "mfma_int8_tops": round(2 * T * k * 2 * n_ff * n_embd / (out["gate_up"] * 1e-6) / 1e12, 2),
                               "mfma_peak_tops": 5000.0}
    res["config"] = (f"prompt path: {T} tokens, top-{k} of {E} NL4 2560 x 768 experts, {layers} layers, "
                     "every expert routed; weights 16 drawn experts tiled over each pool")
    return res


def fit_groups_entries(lines):
    """Least-squares t = a + b n_groups + c n_entries over the sweep lines (b: per expert, c: per
    entry)."""
    import numpy as np
    A = np.array([[1.0, ln["distinct_experts_per_layer"], ln["T"] * 8] for ln in lines])
    t = np.array([ln["us_per_layer_call"] for ln in lines])
    coef, *_ = np.linalg.lstsq(A, t, rcond=None)
    return {"us_fixed": round(float(coef[0]), 3), "us_per_group": round(float(coef[1]), 3),
            "us_per_entry": round(float(coef[2]), 3), "lines": len(lines)}


def profile_for(workload, kind, bytes_per_launch):
    """The committed rocprofv3 kernel-trace summary of `workload` for launch `kind`: its average
    duration and the roofline fraction it gives for `bytes_per_launch`, or None when there is none
    or the kernel sources changed since it was taken."""
    p = os.path.join(ROOT, "profiles", f"kernels_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        doc = json.load(f)
    if doc.get("source_sha256") != source_digest() or kind not in doc.get("kernels", {}):
        return None
    k = doc["kernels"][kind]
    ach = bytes_per_launch / (k["avg_ns"] * 1e-9) / 1e9
    return {"file": f"profiles/kernels_{workload}.md", "avg_launch_us": round(k["avg_ns"] / 1e3, 3),
            "calls": k["calls"], "achieved": round(ach, 1), "frac": round(ach / HBM_PEAK_GBS, 4)}


def traffic_for(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary of `workload`, or None
    when there is none or the kernel sources changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        doc = json.load(f)
    if doc.get("source_sha256") != source_digest():
        return None
    k = doc.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def sweep_line(name, T, routing, steps, warmup, cpu_seconds=0.0, model=None, layout="planar"):
    """One workload's graph-replayed step and launch times (its pools repacked into `layout`);
    with cpu_seconds, the CPU oracle on a sample of its layer calls too (one thread and all
    cores)."""
    import torch

    from moe_routed_expert_route_amd.workloads import Workload
    wl = Workload(name, device="cuda", T=T, routing=routing)
    if layout == "planar":
        wl.to_planar()
    ms_step, _, ks = measure(wl, steps, warmup, reps=5)
    bytes_pass = float(sum(wl.weight_bytes_per_layer()))
    us = ms_step * 1e3 / wl.L
    line = {"T": T, "routing": routing, "layout": layout, "us_per_layer_call": round(us, 3),
            "gbs": round(bytes_pass / (ms_step * 1e-3) / 1e9, 1),
            "distinct_experts_per_layer": round(sum(wl.distinct_experts(l) for l in range(wl.L)) / wl.L, 2),
            "gate_up_us": round(ks["gate_up"], 3), "down_us": round(ks["down"], 3)}
    if cpu_seconds > 0:
        log(f"cpu oracle on {name} T={T}")
        line["cpu_oracle"] = run_cpu_baseline(wl, cpu_seconds, model, layers=4)
    del wl
    torch.cuda.empty_cache()
    return line


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="nl4_2560x768_t1")
    ap.add_argument("--T", type=int, default=None, help="tokens per window (default: the workload's)")
    ap.add_argument("--routing", default=None, help="logits / zipf / uniform / shared (default: the workload's)")
    ap.add_argument("--layout", default="planar", choices=("planar", "rowmajor"),
                    help="weight layout of the timed pools (planar: repacked once at load by moe_repack)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle time to measure")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip the T = 1..4 lines")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the prompt-path line (512 tokens), printed as one JSON line")
    ap.add_argument("--calib", action="store_true",
                    help="first copy 256 MiB device to device (a known-size kernel for counter runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the library "
              "runs on a single GPU (the path would shard by expert ownership, one rank per GPU)",
              file=sys.stderr)
        sys.exit(2)
    model = cpu_model() if not args.no_cpu else None

    import torch

    from moe_routed_expert_route_amd import binding as B
    from moe_routed_expert_route_amd.workloads import Workload

    B.lib()
    torch.cuda.set_device(0)
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_line(reps=args.steps)}), flush=True)
        return
    if args.calib:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("calibration copy: 256 MiB read, 256 MiB written")
    log(f"building workload {args.workload}")
    wl = Workload(args.workload, device="cuda", T=args.T, routing=args.routing, log=log)
    repack = None
    if args.layout == "planar":
        # the row-major pools stay for the alternated layout comparison
        repack = wl.to_planar(keep_rowmajor=not args.no_sweep)
        log(f"repacked every pool into the planar layout ({repack[1] / 1e9:.1f} GB in {repack[0]:.3f} s)")
    per_layer = wl.weight_bytes_per_layer()
    bytes_pass = float(sum(per_layer))
    log(f"pool {wl.pool_bytes / 1e9:.2f} GB, routed bytes per pass {bytes_pass / 1e9:.3f} GB")
    log(f"warmup {args.warmup}, timing {args.steps} steps")
    ms_step, ms_plain, ks = measure(wl, args.steps, args.warmup)
    log("step timed")

    us_layer = ms_step * 1e3 / wl.L
    gbs = bytes_pass / (ms_step * 1e-3) / 1e9
    lb = [wl.launch_bytes(l) for l in range(wl.L)]
    kb = {"gate_up": sum(b[0] for b in lb) / wl.L, "down": sum(b[1] for b in lb) / wl.L}
    fmt_names = {1: "Q8_0", 2: "NL4", 3: "CB2", 4: "CB3", 5: "Q5_1", 6: "NL4X"}
    regw = args.layout == "planar" and wl.fg == 2
    kname = {"gate_up": f"k_gate_up<{fmt_names[wl.fg]}, GU_ROUTED" +
                        (", NL4, true> (weights straight into registers)" if regw else ">"),
             "down": f"k_down<{fmt_names[wl.fd]}>"}
    kernels = {}
    for kind in ("gate_up", "down"):
        avg = ks[kind]
        ach = kb[kind] / (avg * 1e-6) / 1e9
        kernels[kind] = {"kernel": kname[kind], "avg_launch_us": round(avg, 3),
                         "bytes_per_launch": int(kb[kind]),
                         "achieved_gbs": round(ach, 1), "frac": round(ach / HBM_PEAK_GBS, 4)}
    dom = max(kernels, key=lambda k: ks[k])
    dk = kernels[dom]
    traffic = traffic_for(args.workload, dom)
    res = {
        "metric": "us per MoE-layer decode call at T=1..4; expert-weight GB/s (frac of HBM peak)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_replays": {"n": len(wl.last_replays), "median_ms": round(ms_step, 4),
                         "mean_ms": round(sum(wl.last_replays) / len(wl.last_replays), 4),
                         "min_ms": round(min(wl.last_replays), 4), "max_ms": round(max(wl.last_replays), 4)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 dot (v_dot4) with fp32 scales",
        "data": "synthetic (seeded), random-init experts",
        "config": {"workload": f"{wl.L} layers x {wl.E} experts {args.workload}: n_embd {wl.n_embd}, "
                               f"n_ff {wl.n_ff}, top-{wl.k}, T={wl.T}, cold pool "
                               f"{wl.pool_bytes / 1e9:.1f} GB, {args.layout} weight layout",
                   "layout": args.layout,
                   "layers": wl.L, "experts": wl.E, "n_embd": wl.n_embd, "n_ff": wl.n_ff,
                   "top_k": wl.k, "T": wl.T, "parallelism": "single GPU"},
        "us_per_layer_call": round(us_layer, 3),
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "us_per_layer_plain_stream": round(ms_plain * 1e3 / wl.L, 3),
        "roofline": {"bound": "hbm", "kernel": dk["kernel"], "achieved": dk["achieved_gbs"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dk["frac"],
                     "traffic": traffic, "bytes_per_launch": dk["bytes_per_launch"],
                     "avg_launch_us": dk["avg_launch_us"],
                     "profile": profile_for(args.workload, dom, dk["bytes_per_launch"])},
        "kernels": kernels,
    }
    if not args.no_sweep:
        log("two calls per layer")
        res["two_calls_per_layer"] = two_calls_us(wl)
    if not args.no_sweep:
        log("layouts: the row-major and the planar pools alternated")
        if repack is None:
            repack = wl.to_planar(keep_rowmajor=True)
        sec, nb = repack
        wl.use_layout("rowmajor")
        _, _, ks_r = measure(wl, 3, 1)
        graphs = {}
        for name in ("rowmajor", "planar"):
            wl.use_layout(name)
            graphs[name] = step_graph(wl)
        ab = alternate(graphs, rounds=6, per=5)
        del graphs
        wl.use_layout(args.layout)
        res["planar_layout"] = {
            "us_per_layer_call": round(ab["planar"]["median_ms"] * 1e3 / wl.L, 3),
            "us_per_layer_call_rowmajor": round(ab["rowmajor"]["median_ms"] * 1e3 / wl.L, 3),
            "ab": {k: v["visit_medians_ms"] for k, v in ab.items()},
            "rowmajor_gate_up_avg_launch_us": round(ks_r["gate_up"], 3),
            "rowmajor_down_avg_launch_us": round(ks_r["down"], 3),
            "repack_gb": round(nb / 1e9, 3), "repack_s": round(sec, 4),
            "repack_gbs_read_plus_write": round(2 * nb / sec / 1e9, 1),
            "config": "the same workload in both layouts: every pool (all 128 experts of all 48 "
                      "layers) repacked by moe_repack into the planar layout beside the row-major "
                      "pools; step graphs of both alternated A B / B A over 6 rounds of 5 "
                      "replays, medians"}
    if not args.no_cpu:
        res["cpu_baseline"] = run_cpu_baseline(wl, args.cpu_seconds, model)
    del wl
    torch.cuda.empty_cache()
    if not args.no_sweep:
        log("reference streaming read")
        ref = stream_read_gbs()
        res["reference_stream_read"] = ref
        res["frac_of_stream_read"] = round(gbs / ref["gbs"], 4)
        log("empty call")
        res["empty_call"] = empty_call_us()
    if not args.no_sweep:
        sweep = {"nl4_2560x768_shared": [], "cb3q8_2560x640_uniform": []}
        for T in (1, 2, 3, 4):
            log(f"sweep nl4 2560x768 shared experts T={T}")
            sweep["nl4_2560x768_shared"].append(sweep_line("nl4_2560x768_t1", T, "shared", 10, 3))
        t1 = sweep["nl4_2560x768_shared"][0]["us_per_layer_call"]
        for ln in sweep["nl4_2560x768_shared"][1:]:
            ln["per_extra_row_frac_of_t1"] = round((ln["us_per_layer_call"] - t1) / (ln["T"] - 1) / t1, 4)
        # the least-squares slope of t(T) over T = 1..4, as a fraction of t(1)
        import numpy as np
        Ts = np.array([ln["T"] for ln in sweep["nl4_2560x768_shared"]], np.float64)
        ts = np.array([ln["us_per_layer_call"] for ln in sweep["nl4_2560x768_shared"]], np.float64)
        slope = float(((Ts - Ts.mean()) * (ts - ts.mean())).sum() / ((Ts - Ts.mean()) ** 2).sum())
        res["per_extra_row_ls_slope_frac_of_t1"] = round(slope / t1, 4)
        for T in (1, 2, 3, 4):
            log(f"sweep cb3/q8 2560x640 uniform T={T}")
            sweep["cb3q8_2560x640_uniform"].append(
                sweep_line("cb3q8_2560x640", T, "uniform", 10, 3,
                           cpu_seconds=args.cpu_seconds / 2 if T == 4 and not args.no_cpu else 0.0,
                           model=model))
        log("cb2/nl4 T=4 zipf")
        sweep["cb2nl4_2560x768_t4_zipf"] = [
            sweep_line("cb2nl4_2560x768_t4_zipf", 4, "zipf", 10, 3,
                       cpu_seconds=0.0 if args.no_cpu else args.cpu_seconds / 2, model=model)]
        log("nl4/q5_1 T=1")
        sweep["nl4q51_2560x768_t1"] = [sweep_line("nl4q51_2560x768_t1", 1, "logits", 10, 3)]
        log("nl4x T=1")
        sweep["nl4x_2560x768_t1"] = [sweep_line("nl4x_2560x768_t1", 1, "logits", 10, 3)]
        log("prompt path T=512")
        res["prefill"] = prefill_line()
        res["t_sweep"] = sweep
        res["fit_nl4_groups_entries"] = fit_groups_entries(
            sweep["nl4_2560x768_shared"] + sweep["cb2nl4_2560x768_t4_zipf"])
        res["fit_cb3q8_groups_entries"] = fit_groups_entries(sweep["cb3q8_2560x640_uniform"])
    print(json.dumps(res), flush=True)


def cpu_model():
    """The host CPU's model name from lscpu (run before anything touches the GPU), else
    /proc/cpuinfo."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            if line.strip().startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads():
    """Threads for the all-cores oracle run: the cores this process may use, at most
    OMP_NUM_THREADS when that is set (the host's share of cores for this GPU)."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def oracle_calls(wl, layers):
    """A function running the CPU oracle, as it stands, on one whole layer call of the workload
    (route, group, quantize, gate/up, SwiGLU, q8_1, down, scatter) for layer l, with the layer's
    routed experts regenerated on the host beforehand (outside any timing)."""
    import numpy as np

    import oracle
    tb = oracle.Tables(wl.tables["nl4"], wl.tables["cb2"], wl.tables["cb3"])
    ex = {}
    for l in layers:
        ids, _ = oracle.route_topk(wl.logits[l], wl.k)
        ex[l] = {int(e): wl.host_expert(l, int(e)) for e in np.unique(ids)}

    def call(l):
        ids, w = oracle.route_topk(wl.logits[l], wl.k)
        plan = oracle.build_plan(ids, w.astype(np.float32), None, wl.E, 0)
        e = ex[l]
        oracle.layer(wl.x[l], plan, wl.fg, wl.fd, {k: v[0] for k, v in e.items()},
                     {k: v[1] for k, v in e.items()}, {k: v[2] for k, v in e.items()},
                     wl.n_embd, wl.n_ff, np.zeros((wl.T, wl.n_embd), np.float32), tb)
    return call


def time_oracle(call, layers, threads, seconds):
    """(calls, wall seconds): `threads` threads each running layer calls (cycling over `layers`)
    until `seconds` of wall time have passed. The oracle's C routines release the interpreter
    lock, so the threads run on separate cores."""
    import threading
    stop = time.perf_counter() + seconds
    counts = [0] * threads

    def worker(i):
        j = i
        while time.perf_counter() < stop:
            call(layers[j % len(layers)])
            counts[i] += 1
            j += threads
    t0 = time.perf_counter()
    ts = [threading.Thread(target=worker, args=(i,)) for i in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    return sum(counts), time.perf_counter() - t0


def run_cpu_baseline(wl, seconds, model, layers=6, reps=3):
    """The CPU oracle on a bounded sample of the same workload: whole layer calls over `layers`
    of its layers, on one thread and on every core this process may use, each the median of
    `reps` runs of about seconds / (2 reps) each. Weight generation is outside the timed part."""
    lays = list(range(min(layers, wl.L)))
    call = oracle_calls(wl, lays)
    call(lays[0])   # first call: library load and page-in
    n_all = cpu_threads()
    per = seconds / (2 * reps)
    out = {}
    for name, th in (("one_thread", 1), ("all_cores", n_all)):
        us = []
        for _ in range(reps):
            calls, wall = time_oracle(call, lays, th, per)
            us.append(wall / calls * 1e6)
        out[name] = {"us_per_layer_call": round(median(us), 1), "threads": th,
                     "runs_us": [round(u, 1) for u in us]}
    wb = sum(wl.weight_bytes_per_layer()[l] for l in lays) / len(lays)
    return {"value": out["all_cores"]["us_per_layer_call"], "unit": "us per layer call",
            "cores": n_all, "kind": "oracle", "cpu_model": model,
            "one_thread_us_per_layer_call": out["one_thread"]["us_per_layer_call"],
            "runs": out,
            "gbs_all_cores": round(wb / (out["all_cores"]["us_per_layer_call"] * 1e-6) / 1e9, 3),
            "sample": f"whole layer calls of the same workload (same weights, logits and x) over "
                      f"its first {len(lays)} layers: plain-C oracle, float64 sums, as it stands; "
                      f"value = wall time per call with {n_all} threads each running calls (the "
                      f"aggregate rate); one_thread = one thread; each the median of {reps} runs "
                      f"of {per:.1f} s; weight generation excluded"}


if __name__ == "__main__":
    main()
