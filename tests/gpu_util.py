"""Shared helpers of the GPU parity tests: build a seeded workload, run the HIP stages through
the C-ABI, and check each stage against the CPU oracle fed the GPU's own upstream values.

Tolerance (floating point): |gpu - oracle| <= 2e-5 * S, S = sum of |block contributions| of the
element (for Y: |Y0| + sum |w| * S_o); integer and byte results (ids, plan, q8_1 bytes) must be
identical. h is checked to 4 float32 ulps (device expf vs host exp) plus 1e-30 absolute.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from moe_routed_expert_route_amd import binding as B
from moe_routed_expert_route_amd import synth

TOL = 2e-5
NAN_BITS = np.uint32(0x7FC0DEAD)


def dev():
    return torch.device("cuda:0")


def nan_tensor(rows, cols):
    return torch.from_numpy(synth.nan_rows(rows, cols)).to(dev())


class Case:
    """One seeded workload: host weights (only the experts a call touches are generated; every
    other expert pointer aims at a shared zero tensor of the same size), tables, x, plan."""

    def __init__(self, name, n_embd, n_ff, E, fmt_gu, fmt_dn, key, experts_needed):
        self.name, self.n_embd, self.n_ff, self.E = name, n_embd, n_ff, E
        self.fmt_gu, self.fmt_dn = fmt_gu, fmt_dn
        self.tables = oracle.Tables(synth.nl4_table(key), synth.cb2_grid(key), synth.cb3_grid(key))
        need = sorted(set(int(e) for e in experts_needed))
        self.gate, self.up, self.down = {}, {}, {}
        for e in need:
            self.gate[e] = synth.weight_matrix(fmt_gu, n_ff, n_embd, key, e, 0)
            self.up[e] = synth.weight_matrix(fmt_gu, n_ff, n_embd, key, e, 1)
            self.down[e] = synth.weight_matrix(fmt_dn, n_embd, n_ff, key, e, 2)
        d = dev()
        zg = torch.zeros(synth.row_bytes(fmt_gu, n_embd) * n_ff, dtype=torch.uint8, device=d)
        zd = torch.zeros(synth.row_bytes(fmt_dn, n_ff) * n_embd, dtype=torch.uint8, device=d)
        self.dg = {e: torch.from_numpy(self.gate[e]).to(d) for e in need}
        self.du = {e: torch.from_numpy(self.up[e]).to(d) for e in need}
        self.dd = {e: torch.from_numpy(self.down[e]).to(d) for e in need}
        pg = [self.dg[e].data_ptr() if e in self.dg else zg.data_ptr() for e in range(E)]
        pu = [self.du[e].data_ptr() if e in self.du else zg.data_ptr() for e in range(E)]
        pd = [self.dd[e].data_ptr() if e in self.dd else zd.data_ptr() for e in range(E)]
        t64 = dict(dtype=torch.int64, device=d)
        self.layer = B.Layer.from_pointers(
            n_embd, n_ff, fmt_gu, fmt_dn, torch.tensor(pg, **t64), torch.tensor(pu, **t64),
            torch.tensor(pd, **t64),
            nl4=torch.from_numpy(self.tables.nl4).to(d), cb2=torch.from_numpy(self.tables.cb2).to(d),
            cb3=torch.from_numpy(self.tables.cb3).to(d),
            keep=(zg, zd, self.dg, self.du, self.dd))


def planar_twin(c):
    """The same case with every expert matrix repacked on the device (moe_repack) into the planar
    layout and the layer's format fields flagged planar; host weights stay row-major."""
    import copy
    p = copy.copy(c)
    d = dev()
    zg = torch.zeros(synth.row_bytes(c.fmt_gu, c.n_embd) * c.n_ff, dtype=torch.uint8, device=d)
    zd = torch.zeros(synth.row_bytes(c.fmt_dn, c.n_ff) * c.n_embd, dtype=torch.uint8, device=d)
    p.dg = {e: B.moe_repack(c.fmt_gu, t, c.n_ff, c.n_embd) for e, t in c.dg.items()}
    p.du = {e: B.moe_repack(c.fmt_gu, t, c.n_ff, c.n_embd) for e, t in c.du.items()}
    p.dd = {e: B.moe_repack(c.fmt_dn, t, c.n_embd, c.n_ff) for e, t in c.dd.items()}
    pg = [p.dg[e].data_ptr() if e in p.dg else zg.data_ptr() for e in range(c.E)]
    pu = [p.du[e].data_ptr() if e in p.du else zg.data_ptr() for e in range(c.E)]
    pd = [p.dd[e].data_ptr() if e in p.dd else zd.data_ptr() for e in range(c.E)]
    t64 = dict(dtype=torch.int64, device=d)
    L = c.layer
    p.layer = B.Layer.from_pointers(
        c.n_embd, c.n_ff, c.fmt_gu | B.LAYOUT_PLANAR, c.fmt_dn | B.LAYOUT_PLANAR,
        torch.tensor(pg, **t64), torch.tensor(pu, **t64), torch.tensor(pd, **t64),
        nl4=L.nl4, cb2=L.cb2, cb3=L.cb3, keep=(zg, zd, p.dg, p.du, p.dd))
    return p


def offset_twin(c, off):
    """The same case with every expert matrix copied to `off` bytes past a 256-byte boundary (an
    even offset: weight pointers need only 2-byte alignment), the layout kept."""
    import copy
    assert off % 2 == 0
    p = copy.copy(c)
    d = dev()

    def moved(t):
        buf = torch.zeros(t.numel() + 256, dtype=torch.uint8, device=d)
        buf[off:off + t.numel()] = t.reshape(-1).view(torch.uint8)
        return buf

    p.dg = {e: moved(t) for e, t in c.dg.items()}
    p.du = {e: moved(t) for e, t in c.du.items()}
    p.dd = {e: moved(t) for e, t in c.dd.items()}
    zg = torch.zeros(synth.row_bytes(c.fmt_gu & 0xFF, c.n_embd) * c.n_ff + 256, dtype=torch.uint8, device=d)
    zd = torch.zeros(synth.row_bytes(c.fmt_dn & 0xFF, c.n_ff) * c.n_embd + 256, dtype=torch.uint8, device=d)
    pg = [p.dg[e].data_ptr() + off if e in p.dg else zg.data_ptr() for e in range(c.E)]
    pu = [p.du[e].data_ptr() + off if e in p.du else zg.data_ptr() for e in range(c.E)]
    pd = [p.dd[e].data_ptr() + off if e in p.dd else zd.data_ptr() for e in range(c.E)]
    t64 = dict(dtype=torch.int64, device=d)
    L = c.layer
    p.layer = B.Layer.from_pointers(
        c.n_embd, c.n_ff, L.fmt_gate_up, L.fmt_down,
        torch.tensor(pg, **t64), torch.tensor(pu, **t64), torch.tensor(pd, **t64),
        nl4=L.nl4, cb2=L.cb2, cb3=L.cb3, keep=(zg, zd, p.dg, p.du, p.dd))
    return p


def routed_case(name, n_embd, n_ff, E, k, T, fmt_gu, fmt_dn, key, ids=None):
    """Logits routed on the host by the oracle only to know which experts to generate."""
    if ids is None:
        logits = synth.router_logits(T, E, key)
    else:
        logits = synth.logits_for_ids(ids, E, key)
    oids, _ = oracle.route_topk(logits, k)
    c = Case(name, n_embd, n_ff, E, fmt_gu, fmt_dn, key, oids.reshape(-1))
    c.logits, c.k, c.T = logits, k, T
    c.x = synth.activations(T, n_embd, key)
    return c


def gpu_route_and_plan(c, cap_groups, cap_entries, entry_base=0, dst_of_token=None):
    d = dev()
    plan = B.Plan(cap_groups, cap_entries, entry_capacity=entry_base + cap_entries, device=d)
    ids, w = B.moe_route_topk(torch.from_numpy(c.logits).to(d), c.k)
    dst = None if dst_of_token is None else torch.as_tensor(dst_of_token, dtype=torch.int32, device=d)
    B.moe_build_plan(ids, w, plan, c.E, dst_of_token=dst, entry_base=entry_base)
    return plan, ids, w


def run_composed(c, plan, x_np, Y0_np, n_rows, grid_limit=0):
    """quantize -> gate_up -> swiglu -> down_scatter; returns dict of host copies."""
    d = dev()
    x = torch.from_numpy(x_np).to(d)
    xq = B.moe_quantize_q8_1(x)
    ecap = plan.ent_src.numel()
    g = nan_tensor(ecap, c.n_ff)
    u = nan_tensor(ecap, c.n_ff)
    h = nan_tensor(ecap, c.n_ff)
    hq = torch.full((ecap, c.n_ff // 32 * 36), 0xA5, dtype=torch.uint8, device=d)
    B.moe_gate_up(c.layer, plan, xq, g, u, grid_limit=grid_limit)
    B.moe_swiglu_q8_1(plan, g, u, c.n_ff, hq, h=h)
    Y = torch.from_numpy(Y0_np.copy()).to(d)
    B.moe_down_scatter(c.layer, plan, hq, Y, grid_limit=grid_limit)
    torch.cuda.synchronize()
    return dict(xq=xq.cpu().numpy(), g=g.cpu().numpy(), u=u.cpu().numpy(), h=h.cpu().numpy(),
                hq=hq.cpu().numpy(), Y=Y.cpu().numpy(), err=plan.errors())


def run_routed(c, x_np, Y0_np, entry_base=0, dst_of_token=None, grid_limit=0, split=False, step=False,
               ws=None, reps=1):
    """Routing, grouping and the layer step from the logits in two launches (one call, or with
    split=True the two half-step calls, or with step=True the one-launch step, `reps` times on the
    same workspace); returns the plan it published and Y."""
    d = dev()
    T, k = c.T, c.k
    plan = B.Plan(T * k, T * k, entry_capacity=entry_base + T * k, device=d)
    Y = torch.from_numpy(Y0_np.copy()).to(d)
    if ws is None:
        ws = B.workspace(c.layer, plan, device=d)
    dst = None if dst_of_token is None else torch.as_tensor(dst_of_token, dtype=torch.int32, device=d)
    lg, x = torch.from_numpy(c.logits).to(d), torch.from_numpy(x_np).to(d)
    if step:
        for _ in range(reps):
            Y.copy_(torch.from_numpy(Y0_np))
            B.moe_layer_step(c.layer, plan, lg, k, x, Y, ws, dst_of_token=dst, entry_base=entry_base,
                             grid_limit=grid_limit)
    elif split:
        B.moe_layer_gate_up(c.layer, plan, x, ws, logits=lg, k=k, dst_of_token=dst,
                            entry_base=entry_base, grid_limit=grid_limit)
        B.moe_layer_down(c.layer, plan, ws, T, Y, grid_limit=grid_limit)
    else:
        B.moe_layer_decode_routed(c.layer, plan, lg, k, x, Y, ws, dst_of_token=dst,
                                  entry_base=entry_base, grid_limit=grid_limit)
    torch.cuda.synchronize()
    return dict(Y=Y.cpu().numpy(), plan=plan.get(), err=plan.errors())


def run_fused(c, plan, x_np, Y0_np, grid_limit=0, ws=None, stale=False):
    d = dev()
    x = torch.from_numpy(x_np).to(d)
    Y = torch.from_numpy(Y0_np.copy()).to(d)
    if ws is None:
        ws = B.workspace(c.layer, plan, device=d)
    off = B.moe_workspace_layout(c.layer, plan)
    if stale:  # garbage in every byte the call will write and read back
        ws.fill_(0x7F)
    B.moe_layer_decode(c.layer, plan, x, Y, ws, grid_limit=grid_limit)
    torch.cuda.synchronize()
    return dict(Y=Y.cpu().numpy(), ws=ws, off=off, err=plan.errors())


def assert_q81_equal(got, ref, x=None, what="q8_1"):
    """Byte equality of q8_1 rows; on failure name the first differing block and its fields."""
    got = np.asarray(got).reshape(-1, 36)
    ref = np.asarray(ref).reshape(-1, 36)
    bad = np.flatnonzero((got != ref).any(axis=1))
    if bad.size == 0:
        return
    b = int(bad[0])

    def f(r):
        d16 = int(r[0]) | int(r[1]) << 8
        s16 = int(r[2]) | int(r[3]) << 8
        return hex(d16), hex(s16), r[4:].view(np.int8).tolist()
    msg = f"{what}: {bad.size} blocks differ; block {b}: gpu {f(got[b])} oracle {f(ref[b])}"
    if x is not None:
        msg += f" x={np.asarray(x, np.float32).reshape(-1, 32)[b].tolist()}"
    raise AssertionError(msg)


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def check_close(got, ref, S, what):
    got = np.asarray(got, np.float64)
    bad = ~(np.abs(got - ref) <= TOL * S)
    zero_ok = (S == 0) & (got == 0)
    bad &= ~zero_ok
    if bad.any():
        i = np.flatnonzero(bad.reshape(-1))[0]
        raise AssertionError(f"{what}: {bad.sum()} elements out of tolerance; first flat {i}: "
                             f"gpu {got.reshape(-1)[i]!r} ref {ref.reshape(-1)[i]!r} "
                             f"S {S.reshape(-1)[i]!r}")
    return float(np.max(np.abs(got - ref) / np.maximum(S, 1e-300)))


def check_stages(c, plan_host, comp, Y0_np, tables=None):
    """Stage-wise parity of the composed outputs against the oracle fed the GPU's values."""
    tb = tables or c.tables
    base = int(plan_host["entry_base"])
    ng = int(plan_host["n_groups"])
    # S1: q8_1 of x, bytes
    assert_q81_equal(comp["xq"], oracle.quantize_q8_1(c.x), c.x, "xq")
    worst = 0.0
    hq_of = {}
    for gi in range(ng):
        e = int(plan_host["grp_expert"][gi])
        for a in range(int(plan_host["grp_start"][gi]), int(plan_host["grp_start"][gi + 1])):
            src = int(plan_host["ent_src"][a - base])
            xq = comp["xq"][src]
            gr, Sg = oracle.matvec(c.fmt_gu, c.gate[e], c.n_ff, c.n_embd, xq, tb)
            ur, Su = oracle.matvec(c.fmt_gu, c.up[e], c.n_ff, c.n_embd, xq, tb)
            worst = max(worst, check_close(comp["g"][a], gr, Sg, f"g entry {a}"))
            worst = max(worst, check_close(comp["u"][a], ur, Su, f"u entry {a}"))
            # S3: h within 4 ulp of the oracle's SwiGLU on the GPU's g, u
            hr = oracle.swiglu(comp["g"][a], comp["u"][a]).astype(np.float64)
            hg = comp["h"][a].astype(np.float64)
            ulp = np.spacing(np.abs(hr).astype(np.float32)).astype(np.float64)
            assert np.all(np.abs(hg - hr) <= 4 * ulp + 1e-30), f"h entry {a}"
            # S4: hq bytes = oracle q8_1 of the GPU's h
            assert_q81_equal(comp["hq"][a], oracle.quantize_q8_1(comp["h"][a]), comp["h"][a],
                             f"hq entry {a}")
            hq_of[a] = comp["hq"][a]
    # S5: Y from the GPU's hq
    o = oracle.down(plan_host, c.fmt_dn, c.down, c.n_embd, c.n_ff, hq_of, tb)
    Yr, SY = oracle.scatter(plan_host, Y0_np, o)
    written = sorted(set(int(d) for d in plan_host["ent_dst"]))
    if written:
        worst = max(worst, check_close(comp["Y"][written], Yr[written], SY[written], "Y"))
    untouched = [r for r in range(Y0_np.shape[0]) if r not in written]
    assert np.array_equal(bits(comp["Y"][untouched]), bits(Y0_np[untouched])), "untouched Y rows changed"
    return worst


def y0_for(n_rows, n_embd, dst_rows, key):
    """Y0: NaN pattern everywhere, N(0,1) values in the destination rows."""
    Y0 = synth.nan_rows(n_rows, n_embd).copy()
    g = synth.rng(77, key)
    for r in sorted(set(int(d) for d in dst_rows)):
        Y0[r] = g.standard_normal(n_embd).astype(np.float32)
    return Y0
