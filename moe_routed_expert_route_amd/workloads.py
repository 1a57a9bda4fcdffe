"""Device-resident synthetic workloads for the benchmark and the full-size tests.

A workload is a stack of MoE layers, each with its own n_experts experts laid out in one pool
tensor per matrix kind (gate, up, down), so a pass over the layers reads every routed expert
cold from HBM. Inputs come from `synth` (seeded); only the experts the fixed routing selects are
filled with drawn bytes, the rest of the pool is allocated but never read.

Workload shapes are those of the pages' measurements: 2560 x 768 experts ("#363 experts: smaller
and fewer launches for the verify window's PCIe call", "Measured"), 2560 with n_ff 640 ("#2058
Verify window: ...", "What changed"), T = 1..4 windows with top-8 routing.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B
from . import synth

CONFIGS = {
    # 48 layers x 128 experts, NL4 gate/up/down, 2560 x 768, top-8, one token
    "nl4_2560x768_t1": dict(layers=48, E=128, n_embd=2560, n_ff=768, k=8, T=1,
                            fg=synth.NL4, fd=synth.NL4, routing="logits"),
    # same geometry, T = 4 Zipf window, CB2 gate/up, NL4 down
    "cb2nl4_2560x768_t4_zipf": dict(layers=48, E=128, n_embd=2560, n_ff=768, k=8, T=4,
                                    fg=synth.CB2, fd=synth.NL4, routing="zipf"),
    # T sweep geometry: 256 experts, 2560 x 640, CB3 gate/up, Q8_0 down, uniform routing
    # (48 layers: a pass reads >= 0.6 GB, well above the 256 MB last-level cache)
    "cb3q8_2560x640": dict(layers=48, E=256, n_embd=2560, n_ff=640, k=8, T=1,
                           fg=synth.CB3, fd=synth.Q8_0, routing="uniform"),
    # the headline geometry with an offset down format (Q5_1, one of the pages' down formats)
    "nl4q51_2560x768_t1": dict(layers=48, E=128, n_embd=2560, n_ff=768, k=8, T=1,
                               fg=synth.NL4, fd=synth.Q5_1, routing="logits"),
    # the headline geometry in the super-block 4-bit format (4.25 bits per weight)
    "nl4x_2560x768_t1": dict(layers=48, E=128, n_embd=2560, n_ff=768, k=8, T=1,
                             fg=synth.NL4X, fd=synth.NL4X, routing="logits"),
}


def expert_bytes(n_embd, n_ff, fg, fd):
    return 2 * synth.row_bytes(fg, n_embd) * n_ff + synth.row_bytes(fd, n_ff) * n_embd


class Workload:
    def __init__(self, name, device="cuda", T=None, routing=None, layers=None, key=0, log=None):
        cfg = dict(CONFIGS[name])
        if T is not None:
            cfg["T"] = T
        if routing is not None:
            cfg["routing"] = routing
        if layers is not None:
            cfg["layers"] = layers
        self.name, self.cfg = name, cfg
        L, E, n_embd, n_ff, k, T = (cfg[x] for x in ("layers", "E", "n_embd", "n_ff", "k", "T"))
        fg, fd = cfg["fg"], cfg["fd"]
        self.L, self.E, self.n_embd, self.n_ff, self.k, self.T = L, E, n_embd, n_ff, k, T
        self.fg, self.fd = fg, fd
        d = torch.device(device)
        rb_g, rb_d = synth.row_bytes(fg, n_embd), synth.row_bytes(fd, n_ff)
        self.sz_g, self.sz_d = rb_g * n_ff, rb_d * n_embd
        # routing per layer (host logits; the GPU routes them each step)
        self.logits, self.x = [], []
        for l in range(L):
            if cfg["routing"] == "logits":
                lg = synth.router_logits(T, E, key, l)
            else:
                ids = {"zipf": lambda: synth.zipf_ids(T, E, k, 1.1, key, l),
                       "uniform": lambda: synth.uniform_ids(T, E, k, key, l),
                       "shared": lambda: synth.shared_ids(T, E, k, key, l)}[cfg["routing"]]()
                lg = synth.logits_for_ids(ids, E, key, l)
            self.logits.append(lg)
            self.x.append(synth.activations(T, n_embd, key, l))
        self.tables = dict(nl4=synth.nl4_table(key), cb2=synth.cb2_grid(key), cb3=synth.cb3_grid(key))
        # the experts each layer's routing selects (top-k of the logits: the largest k per token)
        self.routed = []
        for lg in self.logits:
            sel = np.argsort(-lg.astype(np.float64), axis=1, kind="stable")[:, :k]
            self.routed.append(sorted(set(int(e) for e in sel.reshape(-1))))
        # pools: one tensor per layer and matrix kind, all experts resident
        self.pool_g, self.pool_u, self.pool_d, self.layers = [], [], [], []
        self.host = {}
        nl4 = torch.from_numpy(self.tables["nl4"]).to(d)
        cb2 = torch.from_numpy(self.tables["cb2"]).to(d)
        cb3 = torch.from_numpy(self.tables["cb3"]).to(d)
        self._tabs = (nl4, cb2, cb3)
        for l in range(L):
            pg = torch.empty(E * self.sz_g, dtype=torch.uint8, device=d)
            pu = torch.empty(E * self.sz_g, dtype=torch.uint8, device=d)
            pd = torch.empty(E * self.sz_d, dtype=torch.uint8, device=d)
            for e in self.routed[l]:
                g = synth.weight_matrix(fg, n_ff, n_embd, key, l, e, 0)
                u = synth.weight_matrix(fg, n_ff, n_embd, key, l, e, 1)
                dn = synth.weight_matrix(fd, n_embd, n_ff, key, l, e, 2)
                pg[e * self.sz_g:(e + 1) * self.sz_g].copy_(torch.from_numpy(g))
                pu[e * self.sz_g:(e + 1) * self.sz_g].copy_(torch.from_numpy(u))
                pd[e * self.sz_d:(e + 1) * self.sz_d].copy_(torch.from_numpy(dn))
            i64 = dict(dtype=torch.int64, device=d)
            ptr_g = torch.tensor([pg.data_ptr() + e * self.sz_g for e in range(E)], **i64)
            ptr_u = torch.tensor([pu.data_ptr() + e * self.sz_g for e in range(E)], **i64)
            ptr_d = torch.tensor([pd.data_ptr() + e * self.sz_d for e in range(E)], **i64)
            lay = B.Layer.from_pointers(n_embd, n_ff, fg, fd, ptr_g, ptr_u, ptr_d, nl4=nl4, cb2=cb2,
                                        cb3=cb3, keep=(pg, pu, pd))
            self.pool_g.append(pg)
            self.pool_u.append(pu)
            self.pool_d.append(pd)
            self.layers.append(lay)
            if log and (l % 8 == 7 or l == L - 1):
                log(f"workload {name}: {l + 1}/{L} layers resident")
        cap = T * k
        self.plans = [B.Plan(cap, cap, device=d) for _ in range(L)]
        self.ids = [torch.empty((T, k), dtype=torch.int32, device=d) for _ in range(L)]
        self.w = [torch.empty((T, k), dtype=torch.float32, device=d) for _ in range(L)]
        self.d_logits = [torch.from_numpy(lg).to(d) for lg in self.logits]
        self.d_x = [torch.from_numpy(x).to(d) for x in self.x]
        self.Y = [torch.zeros((T, n_embd), dtype=torch.float32, device=d) for _ in range(L)]
        self.ws = [B.workspace(self.layers[l], self.plans[l], device=d) for l in range(L)]
        self.pool_bytes = L * E * (2 * self.sz_g + self.sz_d)

    def to_planar(self, keep_rowmajor=False):
        """Repack every pool (all experts of every layer) into the planar layout with moe_repack,
        one pool at a time, and point the layers at the repacked pools with their format fields
        flagged planar. keep_rowmajor: keep the row-major pools and layers too (use_layout switches
        between the two sets). Returns (seconds of repack kernels, bytes read)."""
        if keep_rowmajor:
            self.layouts = {"rowmajor": (list(self.layers), list(self.pool_g), list(self.pool_u),
                                         list(self.pool_d))}
        d = self.pool_g[0].device
        nl4, cb2, cb3 = self._tabs
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ms, nbytes = 0.0, 0
        for l in range(self.L):
            pools = []
            for pool, fmt, rows, cols in ((self.pool_g, self.fg, self.E * self.n_ff, self.n_embd),
                                          (self.pool_u, self.fg, self.E * self.n_ff, self.n_embd),
                                          (self.pool_d, self.fd, self.E * self.n_embd, self.n_ff)):
                dst = torch.empty_like(pool[l])
                ev0.record()
                B.moe_repack(fmt, pool[l], rows, cols, dst=dst, to_planar=True)
                ev1.record()
                torch.cuda.synchronize()
                ms += ev0.elapsed_time(ev1)
                nbytes += pool[l].numel()
                pool[l] = dst
                pools.append(dst)
            pg, pu, pd = pools
            i64 = dict(dtype=torch.int64, device=d)
            ptr_g = torch.tensor([pg.data_ptr() + e * self.sz_g for e in range(self.E)], **i64)
            ptr_u = torch.tensor([pu.data_ptr() + e * self.sz_g for e in range(self.E)], **i64)
            ptr_d = torch.tensor([pd.data_ptr() + e * self.sz_d for e in range(self.E)], **i64)
            self.layers[l] = B.Layer.from_pointers(
                self.n_embd, self.n_ff, self.fg | B.LAYOUT_PLANAR, self.fd | B.LAYOUT_PLANAR,
                ptr_g, ptr_u, ptr_d, nl4=nl4, cb2=cb2, cb3=cb3, keep=(pg, pu, pd))
        if keep_rowmajor:
            self.layouts["planar"] = (list(self.layers), list(self.pool_g), list(self.pool_u),
                                      list(self.pool_d))
        return ms * 1e-3, nbytes

    def use_layout(self, name):
        """Point the layers at the row-major or the planar pools (after to_planar(keep_rowmajor=True))."""
        layers, pg, pu, pd = self.layouts[name]
        self.layers, self.pool_g, self.pool_u, self.pool_d = list(layers), list(pg), list(pu), list(pd)

    # ---------------------------------------------------------------- the step ----------------
    def route_plan(self, l, stream=None):
        B.moe_route_topk(self.d_logits[l], self.k, ids=self.ids[l], w=self.w[l], stream=stream)
        B.moe_build_plan(self.ids[l], self.w[l], self.plans[l], self.E, stream=stream)

    def decode(self, l, stream=None, grid_limit=0):
        B.moe_layer_decode(self.layers[l], self.plans[l], self.d_x[l], self.Y[l], self.ws[l],
                           grid_limit=grid_limit, stream=stream)

    def decode_routed(self, l, stream=None, grid_limit=0):
        B.moe_layer_decode_routed(self.layers[l], self.plans[l], self.d_logits[l], self.k,
                                  self.d_x[l], self.Y[l], self.ws[l], grid_limit=grid_limit,
                                  stream=stream)

    def gate_up(self, l, stream=None):
        """First launch of layer l: route, group, q8_1(x), gate/up, SwiGLU + q8_1 of h."""
        B.moe_layer_gate_up(self.layers[l], self.plans[l], self.d_x[l], self.ws[l],
                            logits=self.d_logits[l], k=self.k, stream=stream)

    def down(self, l, stream=None):
        """Second launch of layer l: grouped down + weighted scatter into Y."""
        B.moe_layer_down(self.layers[l], self.plans[l], self.ws[l], self.T, self.Y[l], stream=stream)

    def step(self, stream=None):
        """One pass of the whole hot path over every layer: route, group, decode (two launches
        per layer: routing and grouping run inside the gate/up launch). The same launches as
        moe_layer_decode_routed, issued through its two halves."""
        for l in range(self.L):
            self.gate_up(l, stream)
            self.down(l, stream)

    def layer_step(self, l, stream=None):
        """Layer l in one launch: route, group, q8_1(x), gate/up, SwiGLU + q8_1, down, scatter."""
        B.moe_layer_step(self.layers[l], self.plans[l], self.d_logits[l], self.k, self.d_x[l], self.Y[l],
                         self.ws[l], stream=stream)

    def step_one_launch(self, stream=None):
        """One pass of the whole hot path over every layer, one launch per layer."""
        for l in range(self.L):
            self.layer_step(l, stream)

    def step_separate(self, stream=None):
        """The same pass with routing and grouping as launches of their own."""
        for l in range(self.L):
            self.route_plan(l, stream)
            self.decode(l, stream)

    # ---------------------------------------------------------------- accounting --------------
    def distinct_experts(self, l):
        return len(self.routed[l])

    def weight_bytes_per_layer(self):
        """Expert-weight bytes each layer call must read: every distinct routed expert once."""
        per = 2 * self.sz_g + self.sz_d
        return [len(r) * per for r in self.routed]

    def launch_bytes(self, l):
        """Algorithmic HBM bytes of layer l's two launches: (gate/up, down). Gate/up reads the
        distinct experts' gate and up matrices once, the logits and x once, and writes the plan,
        the call's descriptor and the q8_1 rows of h (g and u stay on chip); down reads the
        distinct experts' down matrices once, the descriptor, the q8_1 rows of h once and the
        destination rows of Y, and writes those rows."""
        ne = self.T * self.k
        nd = len(self.routed[l])
        hq = ne * (self.n_ff // 32) * 36
        plan = 4 * (2 * nd + 1 + 1 + 3 * ne)
        desc = 4 * (3 + nd + 1 + 3 * ne) + 8 * nd
        gu = nd * 2 * self.sz_g + self.T * self.E * 4 + self.T * self.n_embd * 4 + plan + desc + hq
        dn = nd * self.sz_d + desc + hq + 2 * self.T * self.n_embd * 4
        return gu, dn

    def host_expert(self, l, e):
        """Host copies of one expert's matrices (regenerated from the seed, not read back)."""
        key = 0
        return (synth.weight_matrix(self.fg, self.n_ff, self.n_embd, key, l, e, 0),
                synth.weight_matrix(self.fg, self.n_ff, self.n_embd, key, l, e, 1),
                synth.weight_matrix(self.fd, self.n_embd, self.n_ff, key, l, e, 2))
