"""GPU parity of the HIP path (through the C-ABI) against the CPU oracle, stage by stage.

Workloads (seeded, synthetic; shapes from the pages): the small 8-expert Q8_0 layer; the
2560 x 768 NL4 layer with 128 experts, top-8, T = 1; 2560 x 768 CB2 gate/up + NL4 down with a
T = 4 Zipf window; 2560 x 640 CB3 gate/up + Q8_0 down with 256 experts at T = 1..4 and a window
whose tokens share their experts; 4096 x 1536 Q8_0 plans built directly with 0 / 1 / 2 / 4 / 32
groups, entries from index 7, destinations scattered over 64 NaN-filled rows ("#363 experts:
smaller and fewer launches for the verify window's PCIe call", "Exactness").
"""
import numpy as np
import pytest
import torch

import oracle
from moe_routed_expert_route_amd import binding as B
from moe_routed_expert_route_amd import synth

from . import gpu_util as U

pytestmark = pytest.mark.gpu

Q8_0, NL4, CB2, CB3, Q5_1, NL4X = 1, 2, 3, 4, 5, 6


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    B.lib()


# ------------------------------------------------------------------ quantizer -----------------

def test_quantize_bitexact():
    g = np.random.default_rng(5)
    rows = [g.standard_normal(2560) * s for s in (1.0, 1e-3, 37.0, 2e-7)]
    tie = np.zeros(2560)
    tie[0::32] = 127.0
    tie[1::32] = np.arange(80) - 39.5          # exact k + 1/2 quotients
    rows += [tie, np.zeros(2560)]
    x = np.stack(rows).astype(np.float32)
    q = B.moe_quantize_q8_1(torch.from_numpy(x).to(U.dev()))
    torch.cuda.synchronize()
    U.assert_q81_equal(q.cpu().numpy(), oracle.quantize_q8_1(x), x)


def near_tie_rows(n_rows, n, key):
    """Rows of 32-value blocks whose quotients x / d sit on, or within a few ulp of, k + 1/2 for
    every k in -127..126, under scales that are not powers of two (the division-free quantizer
    must take the division there) and scales outside 2^-100..2^100 (every lane divides)."""
    g = synth.rng(61, key)
    amaxes = [np.float32(v) for v in (100.0, 3.7, 0.013, 1e-20, 1e-35, 1e36, 117.3)]
    out = np.zeros((n_rows, n), np.float32)
    for r in range(n_rows):
        for b in range(n // 32):
            amax = amaxes[(r * 7 + b) % len(amaxes)]
            d = np.float32(amax / np.float32(127.0))
            blk = np.empty(32, np.float32)
            blk[0] = amax if b % 2 else -amax
            ks = g.integers(-127, 127, 31)
            steps = g.integers(-3, 4, 31)
            for i in range(31):
                x = np.float32(np.float32(ks[i] + 0.5) * d)
                for _ in range(abs(int(steps[i]))):
                    x = np.nextafter(x, np.float32(np.inf if steps[i] > 0 else -np.inf), dtype=np.float32)
                blk[1 + i] = np.clip(x, -abs(amax), abs(amax))
            out[r, 32 * b:32 * b + 32] = blk
    return out


def test_quantize_near_ties():
    """Quotients on and next to every half-integer: the quantizer's bytes equal the oracle's (its
    approximate quotient defers to the division there)."""
    x = near_tie_rows(6, 2560, 1)
    q = B.moe_quantize_q8_1(torch.from_numpy(x).to(U.dev()))
    torch.cuda.synchronize()
    U.assert_q81_equal(q.cpu().numpy(), oracle.quantize_q8_1(x), x)


@pytest.mark.parametrize("name", ["nl4_t1", "q8_nl4_t3", "nl4_t4_shared"])
def test_routed_near_tie_x(name):
    """The same rows as x of the routed step: its in-kernel q8_1 of x gives the composed calls' bits
    (whose quantizer the previous test pins to the oracle)."""
    c = _routed(name)
    c.x = near_tie_rows(c.T, c.n_embd, 2)
    n_rows = 8
    dst = np.arange(c.T, dtype=np.int32) + 1
    plan, _, _ = U.gpu_route_and_plan(c, c.T * c.k, c.T * c.k, entry_base=0, dst_of_token=dst)
    Y0 = U.y0_for(n_rows, c.n_embd, dst, 3)
    comp = U.run_composed(c, plan, c.x, Y0, n_rows)
    r = U.run_routed(c, c.x, Y0, entry_base=0, dst_of_token=dst)
    f = U.run_fused(c, plan, c.x, Y0)
    assert comp["err"] == 0 and r["err"] == 0 and f["err"] == 0
    assert np.array_equal(U.bits(r["Y"]), U.bits(comp["Y"]))
    assert np.array_equal(U.bits(f["Y"]), U.bits(comp["Y"]))


def test_swiglu_near_ties():
    """h = silu(30) u = 30 u (1 + e^-30 rounds to 1) placed on and next to half-integer quotients:
    the q8_1 bytes of h equal the oracle's q8_1 of the same h."""
    c = _routed("small_q8")
    plan, _, _ = U.gpu_route_and_plan(c, c.T * c.k, c.T * c.k)
    ecap = plan.ent_src.numel()
    u_np = (near_tie_rows(ecap, c.n_ff, 3) / np.float32(30.0)).astype(np.float32)
    g = torch.full((ecap, c.n_ff), 30.0, dtype=torch.float32, device=U.dev())
    u = torch.from_numpy(u_np).to(U.dev())
    h = torch.full((ecap, c.n_ff), float("nan"), dtype=torch.float32, device=U.dev())
    hq = torch.full((ecap, c.n_ff // 32 * 36), 0xA5, dtype=torch.uint8, device=U.dev())
    B.moe_swiglu_q8_1(plan, g, u, c.n_ff, hq, h=h)
    torch.cuda.synchronize()
    n = int(plan.get()["grp_start"][-1])
    hh = h.cpu().numpy()[:n]
    assert np.array_equal(U.bits(hh), U.bits(oracle.swiglu(g.cpu().numpy()[:n], u_np[:n])))
    U.assert_q81_equal(hq.cpu().numpy()[:n], oracle.quantize_q8_1(hh), hh)


def test_quantize_golden():
    import json
    import os
    doc = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "q8_1_blocks.json")))
    x = np.stack([np.array(b["x"], np.float32) for b in doc["blocks"]])
    q = B.moe_quantize_q8_1(torch.from_numpy(x).to(U.dev())).cpu().numpy()
    for b, row in zip(doc["blocks"], q):
        assert int(row[0]) | int(row[1]) << 8 == int(b["d16"], 16)
        assert int(row[2]) | int(row[3]) << 8 == int(b["s16"], 16)
        assert row[4:].view(np.int8).tolist() == b["q"]


# ------------------------------------------------------------------ route and plan ------------

@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (1, 128, 8), (4, 128, 8), (4, 256, 8), (3, 1000, 32)])
def test_route_topk(T, E, k):
    lg = synth.router_logits(T, E, T, E, k, 1)
    lg[0, 3] = lg[0, 5] = lg[0].max() + 1.0          # a tie at the top: lower id first
    ids, w = B.moe_route_topk(torch.from_numpy(lg).to(U.dev()), k)
    oids, ow = oracle.route_topk(lg, k)
    assert np.array_equal(ids.cpu().numpy(), oids)
    wg = w.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(wg - ow) <= 4 * np.spacing(ow.astype(np.float32)).astype(np.float64))


@pytest.mark.parametrize("T,E,k,base", [(1, 8, 2, 0), (1, 128, 8, 0), (4, 128, 8, 7), (4, 256, 8, 3)])
def test_build_plan(T, E, k, base):
    ids = synth.zipf_ids(T, E, k, 1.1, T, E, base)
    w = synth.rng(31, T).uniform(0.01, 1, (T, k)).astype(np.float32)
    dst = synth.rng(32, T).choice(64, T, replace=False).astype(np.int32)
    plan = B.Plan(T * k, T * k, entry_capacity=base + T * k, device=U.dev())
    d = U.dev()
    B.moe_build_plan(torch.from_numpy(ids).to(d), torch.from_numpy(w).to(d), plan, E,
                     dst_of_token=torch.from_numpy(dst).to(d), entry_base=base)
    got = plan.get()
    ref = oracle.build_plan(ids, w, dst, E, base)
    for key in ("grp_expert", "grp_start", "ent_src", "ent_dst"):
        assert np.array_equal(got[key], ref[key]), key
    assert np.array_equal(U.bits(got["ent_w"]), U.bits(ref["ent_w"]))
    assert got["n_groups"] == ref["n_groups"] and plan.errors() == 0


# ------------------------------------------------------------------ whole step, stage-wise ----

ROUTED = {
    "small_q8": dict(n_embd=256, n_ff=128, E=8, k=2, T=1, fg=Q8_0, fd=Q8_0),
    "nl4_t1": dict(n_embd=2560, n_ff=768, E=128, k=8, T=1, fg=NL4, fd=NL4),
    # tokens sharing their experts: groups of 2 (the register path's largest) and 4 entries on the
    # headline geometry
    "nl4_t2_shared": dict(n_embd=2560, n_ff=768, E=128, k=8, T=2, fg=NL4, fd=NL4, ids="shared"),
    "nl4_t4_shared": dict(n_embd=2560, n_ff=768, E=128, k=8, T=4, fg=NL4, fd=NL4, ids="shared"),
    "cb2_nl4_t4_zipf": dict(n_embd=2560, n_ff=768, E=128, k=8, T=4, fg=CB2, fd=NL4, ids="zipf"),
    "cb3_q8_t2": dict(n_embd=2560, n_ff=640, E=256, k=8, T=2, fg=CB3, fd=Q8_0, ids="uniform"),
    "cb3_q8_t4_shared": dict(n_embd=2560, n_ff=640, E=256, k=8, T=4, fg=CB3, fd=Q8_0, ids="shared"),
    "q8_nl4_t3": dict(n_embd=512, n_ff=256, E=16, k=4, T=3, fg=Q8_0, fd=NL4),
    "nl4_cb2_t2": dict(n_embd=768, n_ff=512, E=16, k=4, T=2, fg=NL4, fd=CB2),
    "cb2_cb3_t4": dict(n_embd=512, n_ff=512, E=12, k=3, T=4, fg=CB2, fd=CB3),
    # groups of 4 entries on rows split over fewer lanes than entries (down: 2 lanes per row)
    "q8_t4_shared_small": dict(n_embd=256, n_ff=128, E=8, k=2, T=4, fg=Q8_0, fd=Q8_0, ids="shared"),
    # 2 units per row: one or two lanes per row
    "nl4_t4_shared_tiny": dict(n_embd=64, n_ff=64, E=4, k=2, T=4, fg=NL4, fd=Q8_0, ids="shared"),
    # many experts: 16 logits per lane in the routing wave, expert pointers past the first 512
    # loaded in a second round, a 32-word selection bitmap
    "q8_e1000_t3": dict(n_embd=256, n_ff=128, E=1000, k=8, T=3, fg=Q8_0, fd=Q8_0),
    # an offset down format: the q8_1 sum field of h enters the down dot product
    "nl4_q51_t1": dict(n_embd=2560, n_ff=768, E=128, k=8, T=1, fg=NL4, fd=Q5_1),
    "cb3_q51_t4_shared": dict(n_embd=512, n_ff=256, E=16, k=4, T=4, fg=CB3, fd=Q5_1, ids="shared"),
    "q8_q51_t3": dict(n_embd=256, n_ff=192, E=8, k=2, T=3, fg=Q8_0, fd=Q5_1),
    # the super-block 4-bit format (NL4 codes, 6-bit sub-block scales)
    "nl4x_t1": dict(n_embd=2560, n_ff=768, E=128, k=8, T=1, fg=NL4X, fd=NL4X),
    "nl4x_q51_t4_zipf": dict(n_embd=512, n_ff=512, E=16, k=4, T=4, fg=NL4X, fd=Q5_1, ids="zipf"),
    "cb2_nl4x_t2": dict(n_embd=768, n_ff=256, E=12, k=3, T=2, fg=CB2, fd=NL4X),
    # the widest one-token window: 4096 columns at 32 lanes a row (two register passes per wave),
    # 64 experts (logits rows padded to the ranking's power of two)
    "nl4_4096_t1": dict(n_embd=4096, n_ff=512, E=64, k=6, T=1, fg=NL4, fd=NL4),
}


def _routed(name, key=0):
    p = ROUTED[name]
    ids = None
    if p.get("ids") == "zipf":
        ids = synth.zipf_ids(p["T"], p["E"], p["k"], 1.1, key)
    elif p.get("ids") == "uniform":
        ids = synth.uniform_ids(p["T"], p["E"], p["k"], key)
    elif p.get("ids") == "shared":
        ids = synth.shared_ids(p["T"], p["E"], p["k"], key)
    return U.routed_case(name, p["n_embd"], p["n_ff"], p["E"], p["k"], p["T"], p["fg"], p["fd"], key,
                         ids=ids)


@pytest.mark.parametrize("name", list(ROUTED))
def test_layer_stages(name):
    c = _routed(name)
    T, k = c.T, c.k
    base = 5
    n_rows = 16
    dst = synth.rng(40, T).choice(n_rows, T, replace=False).astype(np.int32)
    plan, ids, w = U.gpu_route_and_plan(c, T * k, T * k, entry_base=base, dst_of_token=dst)
    ph = plan.get()
    assert np.array_equal(ids.cpu().numpy(), oracle.route_topk(c.logits, k)[0])
    Y0 = U.y0_for(n_rows, c.n_embd, dst, 1)
    comp = U.run_composed(c, plan, c.x, Y0, n_rows)
    assert comp["err"] == 0
    worst = U.check_stages(c, ph, comp, Y0)
    print(f"{name}: worst err/S {worst:.3g}")
    # the single-launch path gives the same bits, and so do its intermediates
    fused = U.run_fused(c, plan, c.x, Y0)
    assert fused["err"] == 0
    assert np.array_equal(U.bits(fused["Y"]), U.bits(comp["Y"]))
    ws, off = fused["ws"].cpu().numpy(), fused["off"]
    ne, nb = int(ph["grp_start"][-1] - base), c.n_ff // 32
    ref = comp["hq"][base:base + ne].reshape(ne, nb, 36)
    lo = ws[off[0]:off[0] + ne * nb * 16].reshape(ne, nb, 16)
    hi = ws[off[1]:off[1] + ne * nb * 16].reshape(ne, nb, 16)
    dq = ws[off[2]:off[2] + ne * nb * 4].view(np.float32).reshape(ne, nb)
    assert np.array_equal(lo, ref[:, :, 4:20]) and np.array_equal(hi, ref[:, :, 20:36])
    d16 = ref[:, :, 0].astype(np.uint16) | (ref[:, :, 1].astype(np.uint16) << 8)
    assert np.array_equal(U.bits(dq), U.bits(d16.view(np.float16).astype(np.float32)))
    if c.fmt_dn == Q5_1:   # the sum fields follow the scales (256-byte aligned)
        so = off[2] + (T * k * nb * 4 + 255) // 256 * 256
        sq = ws[so:so + ne * nb * 4].view(np.float32).reshape(ne, nb)
        s16 = ref[:, :, 2].astype(np.uint16) | (ref[:, :, 3].astype(np.uint16) << 8)
        assert np.array_equal(U.bits(sq), U.bits(s16.view(np.float16).astype(np.float32)))
    # routing + grouping inside the gate/up launch: same plan, same bits
    r = U.run_routed(c, c.x, Y0, entry_base=base, dst_of_token=dst)
    assert r["err"] == 0
    for key in ("n_groups", "grp_expert", "grp_start", "ent_src", "ent_dst"):
        assert np.array_equal(np.asarray(r["plan"][key]), np.asarray(ph[key])), key
    assert np.array_equal(U.bits(r["plan"]["ent_w"]), U.bits(ph["ent_w"]))
    assert np.array_equal(U.bits(r["Y"]), U.bits(comp["Y"]))
    r2 = U.run_routed(c, c.x, Y0, entry_base=base, dst_of_token=dst, split=True)
    assert r2["err"] == 0 and np.array_equal(U.bits(r2["Y"]), U.bits(comp["Y"]))
    # the whole step in one launch (workgroups meet through counts in the workspace), twice on one
    # workspace: the counts are back to zero after each call
    r3 = U.run_routed(c, c.x, Y0, entry_base=base, dst_of_token=dst, step=True, reps=2)
    assert r3["err"] == 0
    for key in ("n_groups", "grp_expert", "grp_start", "ent_src", "ent_dst"):
        assert np.array_equal(np.asarray(r3["plan"][key]), np.asarray(ph[key])), key
    assert np.array_equal(U.bits(r3["Y"]), U.bits(comp["Y"]))


@pytest.mark.parametrize("E,T,k", [(128, 1, 8), (16, 2, 4), (8, 1, 2), (128, 2, 8), (128, 4, 8), (40, 3, 6),
                                   (64, 8, 4), (256, 2, 8)])
def test_routed_ties(E, T, k):
    """Exact ties in the logits through the routed step (the launch ranks the experts itself):
    at the k-th place (the lower id is chosen), inside the chosen set, and a -0 / +0 pair; the
    published plan equals the oracle's routing and grouping, and Y the composed calls' bits."""
    lg = synth.router_logits(T, E, E, T, k, 9) - 3.0
    for t in range(T):
        top = synth.rng(44, E, t).permutation(E)
        lg[t, top[:k + 2]] = np.float32(2.0)                 # k + 2 equal logits: ties at the k-th place
        lg[t, top[0]] = lg[t, top[1]] = np.float32(5.0)      # a tie inside the chosen set
        lg[t, top[2]] = np.float32(0.0)
        lg[t, top[3]] = np.float32(-0.0)                     # equal to +0 (lower id first)
        lg[t, top[4:k + 2]] = np.float32(0.0)
    oids, ow = oracle.route_topk(lg, k)
    need = set(int(e) for e in oids.reshape(-1))
    c = U.Case(f"ties_{E}_{T}", 256, 128, E, Q8_0, Q8_0, 9, need)
    c.logits, c.k, c.T = lg.astype(np.float32), k, T
    c.x = synth.activations(T, 256, 9)
    n_rows = T + 4
    dst = np.arange(T, dtype=np.int32) + 2
    plan, ids, w = U.gpu_route_and_plan(c, T * k, T * k, entry_base=1, dst_of_token=dst)
    assert np.array_equal(ids.cpu().numpy(), oids)
    ph = plan.get()
    ref = oracle.build_plan(oids, ow.astype(np.float32), dst, E, 1)
    for key in ("n_groups", "grp_expert", "grp_start", "ent_src", "ent_dst"):
        assert np.array_equal(np.asarray(ph[key]), np.asarray(ref[key])), key
    Y0 = U.y0_for(n_rows, 256, dst, 2)
    comp = U.run_composed(c, plan, c.x, Y0, n_rows)
    r = U.run_routed(c, c.x, Y0, entry_base=1, dst_of_token=dst)
    assert r["err"] == 0 and comp["err"] == 0
    for key in ("n_groups", "grp_expert", "grp_start", "ent_src", "ent_dst"):
        assert np.array_equal(np.asarray(r["plan"][key]), np.asarray(ph[key])), key
    assert np.array_equal(U.bits(r["plan"]["ent_w"]), U.bits(ph["ent_w"]))
    assert np.array_equal(U.bits(r["Y"]), U.bits(comp["Y"]))


@pytest.mark.parametrize("name", ["q8_nl4_t3", "nl4_t1", "cb2_nl4_t4_zipf"])
def test_two_calls_per_layer(name):
    """One layer as two calls sharing the entry arrays and Y: the even experts' groups first, the
    odd experts' groups second with entries past the first call's. Each call's stages against the
    oracle (the second from the Y the first left); the fused calls give the composed bits, eagerly
    and as a HIP graph of the pair replayed three times."""
    c = _routed(name, key=4)
    T, k = c.T, c.k
    base, n_rows = 3, 8
    dst = synth.rng(41, T).choice(n_rows, T, replace=False).astype(np.int32)
    plan, _, _ = U.gpu_route_and_plan(c, T * k, T * k, entry_base=base, dst_of_token=dst)
    pa, pb = synth.split_plan(plan.get(), lambda e: e % 2 == 0)
    d = U.dev()
    PA = B.Plan(T * k, T * k, entry_capacity=base + T * k, device=d)
    PB = B.Plan(T * k, T * k, entry_capacity=base + T * k, device=d, entries_of=PA)
    PA.set(pa)
    PB.set(pb)
    print(f"{name}: {pa['n_groups']} + {pb['n_groups']} groups", flush=True)
    Y0 = U.y0_for(n_rows, c.n_embd, dst, 2)
    ca = U.run_composed(c, PA, c.x, Y0, n_rows)
    cb = U.run_composed(c, PB, c.x, ca["Y"], n_rows)
    assert ca["err"] == 0 and cb["err"] == 0
    U.check_stages(c, pa, ca, Y0)
    U.check_stages(c, pb, cb, ca["Y"])
    x = torch.from_numpy(c.x).to(d)
    y0 = torch.from_numpy(Y0).to(d)
    Y = y0.clone()
    ws = B.workspace(c.layer, PA, device=d)
    B.moe_layer_decode(c.layer, PA, x, Y, ws)
    B.moe_layer_decode(c.layer, PB, x, Y, ws)
    torch.cuda.synchronize()
    assert np.array_equal(U.bits(Y.cpu().numpy()), U.bits(cb["Y"]))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        B.moe_layer_decode(c.layer, PA, x, Y, ws)
        B.moe_layer_decode(c.layer, PB, x, Y, ws)
    torch.cuda.synchronize()
    for rep in range(3):
        Y.copy_(y0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(U.bits(Y.cpu().numpy()), U.bits(cb["Y"])), rep
    assert PA.errors() == 0
    del g


@pytest.mark.parametrize("fmt,ncols", [(Q8_0, 256), (NL4, 192), (CB2, 768), (CB3, 512), (NL4, 2560),
                                      (Q5_1, 768), (NL4X, 1024)])
def test_repack_bytes(fmt, ncols):
    """moe_repack against the oracle's planar layout, byte for byte, and back."""
    rows = 37
    rb = synth.row_bytes(fmt, ncols)
    m = synth.rng(62, fmt, ncols).integers(0, 256, size=rows * rb, dtype=np.uint8)
    src = torch.from_numpy(m).to(U.dev())
    p = B.moe_repack(fmt, src, rows, ncols, to_planar=True)
    back = B.moe_repack(fmt, p, rows, ncols, to_planar=False)
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy(), oracle.repack(fmt, m, rows, ncols, True))
    assert np.array_equal(back.cpu().numpy(), m)


@pytest.mark.parametrize("name", ["small_q8", "nl4_t1", "nl4_t2_shared", "nl4_t4_shared", "cb2_nl4_t4_zipf", "cb3_q8_t2",
                                  "nl4_cb2_t2", "cb2_cb3_t4", "q8_q51_t3", "nl4x_q51_t4_zipf",
                                  "nl4_t4_shared_tiny", "nl4_4096_t1"])
def test_planar_layer_same_bits(name):
    """Experts repacked into the planar layout give the row-major layer's bits on every path:
    composed (g, u, h, q8_1 of h, Y), fused, routed in two launches, and the one-launch step."""
    c = _routed(name, key=6)
    pc = U.planar_twin(c)
    T, k = c.T, c.k
    base, n_rows = 2, 8
    dst = synth.rng(42, T).choice(n_rows, T, replace=False).astype(np.int32)
    plan, _, _ = U.gpu_route_and_plan(c, T * k, T * k, entry_base=base, dst_of_token=dst)
    Y0 = U.y0_for(n_rows, c.n_embd, dst, 3)
    ref = U.run_composed(c, plan, c.x, Y0, n_rows)
    got = U.run_composed(pc, plan, c.x, Y0, n_rows)
    assert ref["err"] == 0 and got["err"] == 0
    for key in ("g", "u", "h", "Y"):
        assert np.array_equal(U.bits(got[key]), U.bits(ref[key])), key
    assert np.array_equal(got["hq"], ref["hq"])
    f = U.run_fused(pc, plan, c.x, Y0)
    assert f["err"] == 0 and np.array_equal(U.bits(f["Y"]), U.bits(ref["Y"]))
    r = U.run_routed(pc, c.x, Y0, entry_base=base, dst_of_token=dst)
    assert r["err"] == 0 and np.array_equal(U.bits(r["Y"]), U.bits(ref["Y"]))
    r3 = U.run_routed(pc, c.x, Y0, entry_base=base, dst_of_token=dst, step=True)
    assert r3["err"] == 0 and np.array_equal(U.bits(r3["Y"]), U.bits(ref["Y"]))


@pytest.mark.parametrize("name", ["nl4_t1", "nl4_t2_shared"])
def test_planar_skipped_group_same_bits(name):
    """A group whose expert is out of range is skipped (MOE_ERR_EXPERT) the same way on the planar
    NL4 path (weights loaded into registers; a skipped group still issues its count of loads) as on
    the row-major one: fused and composed Y equal bit for bit, rows it owned keep Y0."""
    c = _routed(name, key=8)
    pc = U.planar_twin(c)
    T, k = c.T, c.k
    plan, _, _ = U.gpu_route_and_plan(c, T * k, T * k)
    Y0 = U.y0_for(T, c.n_embd, range(T), 6)
    plan.grp_expert[1] = 100000                  # out of range: group 1 skipped in both launches
    for run in (lambda cc: U.run_fused(cc, plan, c.x, Y0),
                lambda cc: U.run_composed(cc, plan, c.x, Y0, T)):
        plan.err.zero_()
        ref = run(c)
        assert ref["err"] & 4
        plan.err.zero_()
        got = run(pc)
        assert got["err"] & 4
        assert np.array_equal(U.bits(got["Y"]), U.bits(ref["Y"]))


@pytest.mark.parametrize("name,planar,off", [("nl4_t1", True, 2), ("nl4_t1", True, 6), ("nl4_t2_shared", True, 10),
                                             ("nl4_t4_shared", True, 2), ("nl4_t1", False, 2)])
def test_unaligned_experts_same_bits(name, planar, off):
    """Expert matrices that start 2, 6 or 10 bytes past a 16-byte boundary (weight pointers need
    only 2-byte alignment) give the aligned layer's bits on every path: the planar register loads
    then read unaligned 16-byte pieces, and the LDS passes take the realigning reads."""
    c = _routed(name, key=11)
    ref_case = U.planar_twin(c) if planar else c
    moved = U.offset_twin(ref_case, off)
    T, k = c.T, c.k
    base, n_rows = 1, 8
    dst = synth.rng(43, T).choice(n_rows, T, replace=False).astype(np.int32)
    plan, _, _ = U.gpu_route_and_plan(c, T * k, T * k, entry_base=base, dst_of_token=dst)
    Y0 = U.y0_for(n_rows, c.n_embd, dst, 4)
    ref = U.run_composed(ref_case, plan, c.x, Y0, n_rows)
    got = U.run_composed(moved, plan, c.x, Y0, n_rows)
    assert ref["err"] == 0 and got["err"] == 0
    for key in ("g", "u", "h", "Y"):
        assert np.array_equal(U.bits(got[key]), U.bits(ref[key])), key
    f = U.run_fused(moved, plan, c.x, Y0)
    assert f["err"] == 0 and np.array_equal(U.bits(f["Y"]), U.bits(ref["Y"]))
    r = U.run_routed(moved, c.x, Y0, entry_base=base, dst_of_token=dst)
    assert r["err"] == 0 and np.array_equal(U.bits(r["Y"]), U.bits(ref["Y"]))


@pytest.mark.parametrize("name,planar", [("nl4_t1", False), ("cb2_nl4_t4_zipf", False), ("nl4_t1", True),
                                         ("nl4_t2_shared", True), ("nl4_t4_shared", True)])
def test_grid_invariance(name, planar):
    """Every path and every grid limit gives the same bits (planar NL4: each wave may take several
    passes, each loaded into registers on its own)."""
    c = _routed(name, key=2)
    if planar:
        c = U.planar_twin(c)
    T, k = c.T, c.k
    plan, _, _ = U.gpu_route_and_plan(c, T * k, T * k)
    Y0 = U.y0_for(T, c.n_embd, range(T), 3)
    ref = U.run_fused(c, plan, c.x, Y0)["Y"]
    comp = U.run_composed(c, plan, c.x, Y0, T)["Y"]
    assert np.array_equal(U.bits(ref), U.bits(comp))
    for gl in (1, 2, 3, 4, T * k, 5000):
        y = U.run_fused(c, plan, c.x, Y0, grid_limit=gl)["Y"]
        assert np.array_equal(U.bits(y), U.bits(ref)), gl
        y2 = U.run_composed(c, plan, c.x, Y0, T, grid_limit=gl)["Y"]
        assert np.array_equal(U.bits(y2), U.bits(ref)), gl
        y3 = U.run_routed(c, c.x, Y0, grid_limit=gl)["Y"]
        assert np.array_equal(U.bits(y3), U.bits(ref)), gl
        r4 = U.run_routed(c, c.x, Y0, grid_limit=gl, step=True)
        assert r4["err"] == 0 and np.array_equal(U.bits(r4["Y"]), U.bits(ref)), gl


# ------------------------------------------------------------------ edge matrix ---------------

_C5 = {}


def _c5_case(ng):
    if ng not in _C5:
        p = synth.direct_plan(ng, 256, 4, 64, 7, 5, max_entries=32)
        c = U.Case(f"c5_{ng}", 4096, 1536, 256, Q8_0, Q8_0, 5, p["grp_expert"])
        c.x = synth.activations(4, 4096, 5, ng)
        _C5[ng] = (c, p)
    return _C5[ng]


@pytest.mark.parametrize("ng", [0, 1, 2, 4, 32])
def test_edges_q8_4096(ng):
    c, p = _c5_case(ng)
    plan = B.Plan(32, 32, entry_capacity=7 + 32, device=U.dev())
    plan.set(p)
    Y0 = U.y0_for(64, 4096, p["ent_dst"], 9)
    comp = U.run_composed(c, plan, c.x, Y0, 64)
    assert comp["err"] == 0
    if ng == 0:
        assert np.array_equal(U.bits(comp["Y"]), U.bits(Y0))
    else:
        U.check_stages(c, p, comp, Y0)
    # entries past index 0: rows 0..6 of g / u / hq are never written
    assert np.array_equal(U.bits(comp["g"][:7]), np.full((7, 1536), U.NAN_BITS, np.uint32))
    assert np.all(comp["hq"][:7] == 0xA5)
    fused = U.run_fused(c, plan, c.x, Y0, stale=True)
    assert np.array_equal(U.bits(fused["Y"]), U.bits(comp["Y"]))
    for gl in (1, 3, 4, 33):
        assert np.array_equal(U.bits(U.run_fused(c, plan, c.x, Y0, grid_limit=gl)["Y"]),
                              U.bits(comp["Y"])), gl


@pytest.mark.parametrize("fmt,planar", [(Q8_0, False), (NL4, True)])
def test_one_token_plan_with_repeated_entries(fmt, planar):
    """A caller's plan for one token whose groups hold 1, 2 and 3 entries (the token chosen again,
    to different rows): the one-token down launch takes one pass per entry; the fused call gives
    the composed calls' bits, and the stages hold against the oracle."""
    n_embd, n_ff = (2560, 768) if fmt == NL4 else (512, 256)
    exps = np.array([3, 7, 11], np.int32)
    c = U.Case(f"rep_{fmt}", n_embd, n_ff, 16, fmt, fmt, 12, exps)
    c.x = synth.activations(1, n_embd, 12)
    p = dict(n_groups=3, grp_expert=exps, grp_start=np.array([4, 5, 7, 10], np.int32), entry_base=4,
             ent_src=np.zeros(6, np.int32), ent_dst=np.array([2, 2, 5, 2, 5, 7], np.int32),
             ent_w=np.array([0.3, 0.7, 0.2, 0.9, 0.45, 0.6], np.float32), T=1)
    plan = B.Plan(4, 8, entry_capacity=4 + 8, device=U.dev())
    plan.set(p)
    cc = U.planar_twin(c) if planar else c
    Y0 = U.y0_for(8, n_embd, p["ent_dst"], 7)
    comp = U.run_composed(cc, plan, c.x, Y0, 8)
    assert comp["err"] == 0
    U.check_stages(c, p, comp, Y0)
    fused = U.run_fused(cc, plan, c.x, Y0)
    assert fused["err"] == 0 and np.array_equal(U.bits(fused["Y"]), U.bits(comp["Y"]))


# (matrix, byte offset in the expert's Q8_0 matrix, bits): Q8_0 block = fp16 d (bytes 0-1), 32 quants
CORRUPT = {
    "gate_quant": ("gate", 34 * 3 + 2, 0x40),     # row 0, block 3, quant 0
    "gate_scale": ("gate", 34 * 3 + 1, 0x04),     # row 0, block 3, an exponent bit of d
    "up_scale": ("up", 34 * 5 + 0, 0x80),         # row 0, block 5, a mantissa bit of d
    "down_scale": ("down", 34 * 2 + 1, 0x08),     # row 0, block 2, an exponent bit of d
}


@pytest.mark.parametrize("where", list(CORRUPT))
def test_negative_corrupted_weight_is_caught(where):
    """A byte flipped in the oracle's copy of one expert (a quant or a scale of a gate, up or down
    matrix) must fail the parity check of the GPU's unchanged results."""
    c = _routed("small_q8", key=3)
    plan, _, _ = U.gpu_route_and_plan(c, 2, 2)
    ph = plan.get()
    Y0 = U.y0_for(1, c.n_embd, [0], 4)
    comp = U.run_composed(c, plan, c.x, Y0, 1)
    U.check_stages(c, ph, comp, Y0)
    e = int(ph["grp_expert"][0])
    mat, off, bit = CORRUPT[where]
    bad = getattr(c, mat)[e].copy()
    bad[off] ^= bit
    getattr(c, mat)[e] = bad
    with pytest.raises(AssertionError):
        U.check_stages(c, ph, comp, Y0)


def test_offset_format_rejected_for_gate_up():
    """Q5_1 is a down format only: a layer naming it for gate/up is refused on the host."""
    c = _routed("q8_q51_t3", key=7)
    L = c.layer
    bad = B.Layer.from_pointers(c.n_embd, c.n_ff, Q5_1, Q5_1, L.ptr_gate, L.ptr_up, L.ptr_down)
    plan, _, _ = U.gpu_route_and_plan(c, c.T * c.k, c.T * c.k)
    xq = B.moe_quantize_q8_1(torch.from_numpy(c.x).to(U.dev()))
    g = torch.empty((c.T * c.k, c.n_ff), dtype=torch.float32, device=U.dev())
    with pytest.raises(RuntimeError, match="unknown weight format"):
        B.moe_gate_up(bad, plan, xq, g, g.clone())


def test_device_errors_reported():
    c = _routed("small_q8", key=4)
    plan, _, _ = U.gpu_route_and_plan(c, 2, 2)
    Y0 = U.y0_for(1, c.n_embd, [0], 5)
    plan.n_groups.fill_(3)                       # above cap_groups
    r = U.run_fused(c, plan, c.x, Y0)
    assert r["err"] & 1 and np.array_equal(U.bits(r["Y"]), U.bits(Y0))
    plan.err.zero_()
    plan.n_groups.fill_(2)
    plan.grp_expert[1] = 99                      # expert out of range: that group skipped
    r = U.run_fused(c, plan, c.x, Y0)
    assert r["err"] & 4
    plan.err.zero_()
    plan.grp_expert[1] = int(plan.get()["grp_expert"][0]) + 1
    plan.ent_dst[0] = 50                          # destination out of range: entry skipped
    r = U.run_fused(c, plan, c.x, Y0)
    assert r["err"] & 16
