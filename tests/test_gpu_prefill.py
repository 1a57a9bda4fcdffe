"""Prompt path (many tokens, matrix cores) against the oracle, through the C-ABI.

The chain is moe_quantize_q8_1 -> moe_prefill_plan -> moe_prefill_gate_up ->
moe_prefill_swiglu_q8_1 -> moe_prefill_down -> moe_prefill_scatter. The plan is compared with the
oracle's grouping bit for bit (and the choice -> entry map with its inverse); every stage's values
are checked against the oracle fed the GPU's upstream values, to the decode path's tolerance
(2e-5 of the sum of |block contributions|; h within 4 float32 ulps; q8_1 bytes exact); the rows of
Y that no token names keep their NaN pattern.
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

PREFILL = {
    # groups of about 16 entries (a ragged second 16-entry tile), one K chunk
    "q8_t64": dict(n_embd=256, n_ff=256, E=8, k=2, T=64, fg=Q8_0, fd=Q8_0),
    # a ragged K chunk (576 = 512 + 64 weights), groups past one 32-entry pass
    "nl4_t96_e8": dict(n_embd=576, n_ff=384, E=8, k=4, T=96, fg=NL4, fd=NL4),
    "cb2_q51_t40": dict(n_embd=512, n_ff=256, E=16, k=4, T=40, fg=CB2, fd=Q5_1),
    "cb3_nl4x_t33": dict(n_embd=768, n_ff=512, E=12, k=3, T=33, fg=CB3, fd=NL4X),
    "nl4x_q8_t50": dict(n_embd=1024, n_ff=320, E=24, k=4, T=50, fg=NL4X, fd=Q8_0),
    # the decode geometry with a prompt's worth of tokens
    "nl4_2560x768_t24": dict(n_embd=2560, n_ff=768, E=128, k=8, T=24, fg=NL4, fd=NL4),
    # about 80 entries per group: every group takes a second 64-entry pass over its rows
    "nl4_t160_e4": dict(n_embd=512, n_ff=256, E=4, k=2, T=160, fg=NL4, fd=NL4),
}

# the benchmarked prompt-path shape: 512 tokens, top-8 of 128 NL4 experts of 2560 x 768 (every
# expert routed, about 32 entries per group: many 32-entry passes over five K chunks of 512)
BENCH = dict(n_embd=2560, n_ff=768, E=128, k=8, T=512, fg=NL4, fd=NL4)


def _case(name, key=0):
    p = PREFILL[name]
    return U.routed_case(name, p["n_embd"], p["n_ff"], p["E"], p["k"], p["T"], p["fg"], p["fd"], key)


def _plan(c, base, dst):
    d = U.dev()
    n = c.T * c.k
    plan = B.Plan(min(c.E, n), n, entry_capacity=base + n, device=d)
    ids, w = B.moe_route_topk(torch.from_numpy(c.logits).to(d), c.k)
    dt = torch.as_tensor(dst, dtype=torch.int32, device=d)
    ent_of = B.moe_prefill_plan(ids, w, plan, c.E, dst_of_token=dt, entry_base=base)
    return plan, ids, w, ent_of, dt


@pytest.mark.parametrize("name", list(PREFILL))
def test_prefill_stages(name):
    c = _case(name)
    T, k, d = c.T, c.k, U.dev()
    base, n_rows = 3, T + 5
    dst = synth.rng(43, T).permutation(n_rows)[:T].astype(np.int32)
    plan, ids, w, ent_of, dt = _plan(c, base, dst)
    ph = plan.get()
    ref = oracle.build_plan(ids.cpu().numpy(), w.cpu().numpy(), dst, c.E, base)
    for key in ("n_groups", "grp_expert", "grp_start", "ent_src", "ent_dst"):
        assert np.array_equal(np.asarray(ph[key]), np.asarray(ref[key])), key
    assert np.array_equal(U.bits(ph["ent_w"]), U.bits(ref["ent_w"]))
    eo, ids_h = ent_of.cpu().numpy(), ids.cpu().numpy()
    for t in range(T):   # ent_of names each choice's entry: its token and its expert
        for j in range(k):
            a = int(eo[t, j]) - base
            g = int(np.searchsorted(ph["grp_start"], eo[t, j], "right")) - 1
            assert ph["ent_src"][a] == t and ph["grp_expert"][g] == ids_h[t, j]
    ecap = base + T * k
    xq = B.moe_quantize_q8_1(torch.from_numpy(c.x).to(d))
    g = U.nan_tensor(ecap, c.n_ff)
    u = U.nan_tensor(ecap, c.n_ff)
    h = U.nan_tensor(ecap, c.n_ff)
    hq = torch.full((ecap, c.n_ff // 32 * 36), 0xA5, dtype=torch.uint8, device=d)
    B.moe_prefill_gate_up(c.layer, plan, xq, g, u)
    B.moe_prefill_swiglu_q8_1(plan, g, u, c.n_ff, hq, h=h)
    O = U.nan_tensor(ecap, c.n_embd)
    B.moe_prefill_down(c.layer, plan, hq, O)
    Y0 = U.y0_for(n_rows, c.n_embd, dst, 4)
    Y = torch.from_numpy(Y0.copy()).to(d)
    B.moe_prefill_scatter(plan, ent_of, O, Y, c.n_embd, dst_of_token=dt)
    torch.cuda.synchronize()
    assert plan.errors() == 0
    comp = dict(xq=xq.cpu().numpy(), g=g.cpu().numpy(), u=u.cpu().numpy(), h=h.cpu().numpy(),
                hq=hq.cpu().numpy(), Y=Y.cpu().numpy())
    worst = U.check_stages(c, ph, comp, Y0)
    print(f"{name}: {ph['n_groups']} groups, worst err/S {worst:.3g}")


def test_prefill_plan_large():
    """16384 choices (2048 tokens x top-8 of 128): the plan and the choice -> entry map equal the
    oracle's grouping bit for bit, with entries from past 0."""
    T, E, k, base = 2048, 128, 8, 11
    d = U.dev()
    logits = synth.router_logits(T, E, 17)
    ids, w = B.moe_route_topk(torch.from_numpy(logits).to(d), k)
    plan = B.Plan(E, T * k, entry_capacity=base + T * k, device=d)
    ent_of = B.moe_prefill_plan(ids, w, plan, E, entry_base=base)
    ph = plan.get()
    ref = oracle.build_plan(ids.cpu().numpy(), w.cpu().numpy(), None, E, base)
    for key in ("n_groups", "grp_expert", "grp_start", "ent_src", "ent_dst"):
        assert np.array_equal(np.asarray(ph[key]), np.asarray(ref[key])), key
    assert np.array_equal(U.bits(ph["ent_w"]), U.bits(ref["ent_w"]))
    eo = ent_of.cpu().numpy().reshape(-1) - base
    assert np.array_equal(np.sort(eo), np.arange(T * k))   # a bijection onto the entries
    assert np.array_equal(ph["ent_src"][eo], np.repeat(np.arange(T), k))
    assert plan.errors() == 0


def test_prefill_bench_shape():
    """The prompt path at the shape the benchmark times, launched as it launches it (entries from
    0, each token its own destination row): the plan bit for bit, x's q8_1 bytes for every token,
    and g, u, h, hq, the per-entry down rows O and Y element by element on a seeded sample of 48
    tokens (their 384 entries), each against the oracle fed the GPU's upstream values."""
    p = BENCH
    c = U.routed_case("prefill_bench", p["n_embd"], p["n_ff"], p["E"], p["k"], p["T"], p["fg"], p["fd"], 5)
    T, k, d, n = c.T, c.k, U.dev(), c.T * c.k
    plan = B.Plan(c.E, n, device=d)
    ids, w = B.moe_route_topk(torch.from_numpy(c.logits).to(d), k)
    ent_of = B.moe_prefill_plan(ids, w, plan, c.E)
    ph = plan.get()
    ref = oracle.build_plan(ids.cpu().numpy(), w.cpu().numpy(), None, c.E, 0)
    for key in ("n_groups", "grp_expert", "grp_start", "ent_src", "ent_dst"):
        assert np.array_equal(np.asarray(ph[key]), np.asarray(ref[key])), key
    assert np.array_equal(U.bits(ph["ent_w"]), U.bits(ref["ent_w"]))
    sizes = np.diff(ph["grp_start"])
    assert ph["n_groups"] == c.E and sizes.max() > 32, sizes
    xq = B.moe_quantize_q8_1(torch.from_numpy(c.x).to(d))
    g = torch.empty((n, c.n_ff), dtype=torch.float32, device=d)
    u = torch.empty_like(g)
    h = torch.empty_like(g)
    hq = torch.empty((n, c.n_ff // 32 * 36), dtype=torch.uint8, device=d)
    O = torch.empty((n, c.n_embd), dtype=torch.float32, device=d)
    Y0 = synth.rng(78, T).standard_normal((T, c.n_embd)).astype(np.float32)
    Y = torch.from_numpy(Y0.copy()).to(d)
    B.moe_prefill_gate_up(c.layer, plan, xq, g, u)
    B.moe_prefill_swiglu_q8_1(plan, g, u, c.n_ff, hq, h=h)
    B.moe_prefill_down(c.layer, plan, hq, O)
    B.moe_prefill_scatter(plan, ent_of, O, Y, c.n_embd)
    torch.cuda.synchronize()
    assert plan.errors() == 0
    xq_h = xq.cpu().numpy()
    U.assert_q81_equal(xq_h, oracle.quantize_q8_1(c.x), c.x, "xq")
    g_h, u_h, h_h, hq_h = g.cpu().numpy(), u.cpu().numpy(), h.cpu().numpy(), hq.cpu().numpy()
    O_h, Y_h, eo = O.cpu().numpy(), Y.cpu().numpy(), ent_of.cpu().numpy()
    ids_h = ids.cpu().numpy()
    group_of = np.searchsorted(ph["grp_start"], np.arange(n), "right") - 1
    worst = 0.0
    for t in sorted(synth.rng(79).choice(T, 48, replace=False)):
        yr = Y0[t].astype(np.float64)
        sy = np.abs(yr)
        for j in range(k):
            a = int(eo[t, j])
            e = int(ph["grp_expert"][group_of[a]])
            assert ph["ent_src"][a] == t and e == ids_h[t, j]
            gr, Sg = oracle.matvec(c.fmt_gu, c.gate[e], c.n_ff, c.n_embd, xq_h[t], c.tables)
            ur, Su = oracle.matvec(c.fmt_gu, c.up[e], c.n_ff, c.n_embd, xq_h[t], c.tables)
            worst = max(worst, U.check_close(g_h[a], gr, Sg, f"g entry {a}"))
            worst = max(worst, U.check_close(u_h[a], ur, Su, f"u entry {a}"))
            hr = oracle.swiglu(g_h[a], u_h[a]).astype(np.float64)
            ulp = np.spacing(np.abs(hr).astype(np.float32)).astype(np.float64)
            assert np.all(np.abs(h_h[a].astype(np.float64) - hr) <= 4 * ulp + 1e-30), f"h entry {a}"
            U.assert_q81_equal(hq_h[a], oracle.quantize_q8_1(h_h[a]), h_h[a], f"hq entry {a}")
            o, So = oracle.matvec(c.fmt_dn, c.down[e], c.n_embd, c.n_ff, hq_h[a], c.tables)
            wa = float(ph["ent_w"][a])
            worst = max(worst, U.check_close(O_h[a], wa * o, abs(wa) * So, f"O entry {a}"))
            yr = yr + wa * o
            sy = sy + abs(wa) * So
        worst = max(worst, U.check_close(Y_h[t], yr, sy, f"Y row {t}"))
    print(f"prefill bench shape: {ph['n_groups']} groups, largest {sizes.max()} entries, "
          f"worst err/S {worst:.3g}")
