"""Pins of the oracle's router, plan builder, SwiGLU and whole-layer loop (CPU only).

Router: softmax over the expert logits, top-k, weights renormalised over the k (the workload's
routing recipe); ids are pinned to numpy.lexsort, weights to scipy.special.softmax over the
selected logits (renormalising a softmax over a subset equals the softmax of that subset).
Plan: entries grouped by expert ("#2058 Verify window: ...", "Why": each expert's weights are
decoded once and applied to the group's entries), groups ascending by expert, entries ascending
by token, absolute indices from entry_base ("#363 experts: ...", "Exactness": entries from past 0).
SwiGLU: silu(gate) * up in float32, one rounding per operation (expf, 1 + e, g / den, s * u;
"#363 ...", "What changes": the product is rounded on its own); pinned to closed forms, to
scipy.special.expit in float64 within the error bound of four float32 roundings, and to crafted
inputs on which that order and a float64 evaluation rounded once give different floats.
Layer: brute force on the small workload (8 experts, 256 x 128, top-2, Q8_0) against a dense
float64 numpy formula built from dequantized weights and quantized activations.
"""
import math

import numpy as np
import pytest
from scipy.special import expit, softmax

from moe_routed_expert_route_amd import synth

from .test_oracle_decode import np_dequant, np_dequant_q8_1

Q8_0, NL4, CB2, CB3 = 1, 2, 3, 4


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (4, 128, 8), (3, 256, 8), (2, 16, 16)])
def test_route_topk(orc, T, E, k):
    lg = synth.router_logits(T, E, T, E, k)
    ids, w = orc.route_topk(lg, k)
    for t in range(T):
        order = np.lexsort((np.arange(E), -lg[t].astype(np.float64)))[:k]
        assert ids[t].tolist() == order.tolist()
        ref = softmax(lg[t, ids[t]].astype(np.float64))
        assert np.allclose(w[t], ref, rtol=1e-13, atol=0)
        assert abs(w[t].sum() - 1.0) < 1e-14
    if k == E:
        assert np.allclose(np.take_along_axis(w, np.argsort(ids, 1), 1), softmax(lg.astype(np.float64), axis=1),
                           rtol=1e-13)


def test_route_ties_lower_id_first(orc):
    lg = np.zeros((1, 8), np.float32)
    lg[0, [5, 2, 7]] = 1.0
    ids, w = orc.route_topk(lg, 2)
    assert ids[0].tolist() == [2, 5]
    assert np.allclose(w[0], [0.5, 0.5])


def test_logits_for_ids_route_back(orc):
    ids = synth.zipf_ids(4, 128, 8, 1.1, 3)
    lg = synth.logits_for_ids(ids, 128, 3)
    got, _ = orc.route_topk(lg, 8)
    assert np.array_equal(np.sort(got, 1), np.sort(ids, 1))


@pytest.mark.parametrize("T,E,k,base", [(1, 8, 2, 0), (4, 128, 8, 7), (4, 256, 8, 0), (3, 16, 4, 100)])
def test_build_plan(orc, T, E, k, base):
    ids = synth.zipf_ids(T, E, k, 1.1, T, E) if E >= k else None
    w = synth.rng(9, T).uniform(0, 1, (T, k)).astype(np.float32)
    dst = synth.rng(10, T).choice(64, T, replace=False).astype(np.int32)
    p = orc.build_plan(ids, w, dst, E, base)
    ng = p["n_groups"]
    ge, gs = p["grp_expert"], p["grp_start"]
    cnt = np.bincount(ids.reshape(-1), minlength=E)
    assert ng == np.count_nonzero(cnt)
    assert ge.tolist() == np.flatnonzero(cnt).tolist()             # ascending experts
    assert gs[0] == base and gs[-1] == base + T * k
    assert np.diff(gs).tolist() == cnt[ge].tolist()
    seen = set()
    for gi in range(ng):
        toks = p["ent_src"][gs[gi] - base: gs[gi + 1] - base]
        assert np.all(np.diff(toks) > 0)                             # ascending tokens
        for t in toks:
            j = ids[t].tolist().index(ge[gi])
            seen.add((int(t), j))
            r = list(range(gs[gi] - base, gs[gi + 1] - base))[list(toks).index(t)]
            assert p["ent_w"][r] == w[t, j] and p["ent_dst"][r] == dst[t]
    assert len(seen) == T * k                                        # a permutation of entries


def test_build_plan_rejects_bad_id(orc):
    with pytest.raises(ValueError):
        orc.build_plan(np.array([[0, 9]], np.int32), None, None, 8, 0)


def test_swiglu(orc):
    g = np.array([0.0, -0.0, 100.0, -200.0, 1.0, -1.0, 3.5, 1e-30], np.float32)
    u = np.array([2.0, 2.0, 0.5, 3.0, 1.0, 1.0, -2.0, 1.0], np.float32)
    h = orc.swiglu(g, u)
    assert h[0] == 0.0 and h[2] == np.float32(50.0)
    assert h[3] == 0.0                      # expf(200) overflows: -200 / inf * 3 = -0
    rng = np.random.default_rng(4)
    g2 = (rng.standard_normal(20000) * 4).astype(np.float32)
    u2 = rng.standard_normal(20000).astype(np.float32)
    ref = (g2.astype(np.float64) * expit(g2.astype(np.float64))) * u2.astype(np.float64)
    got = orc.swiglu(g2, u2).astype(np.float64)
    # four roundings to float32 (expf within half an ulp and a little, the add, the divide, the
    # multiply; the error of expf enters the sum scaled by e / (1 + e) < 1): relative error at
    # most about 4 * 2^-24, i.e. under 4 ulp, plus the subnormal quantum
    assert np.all(np.abs(got - ref) <= 4.01 * 2.0 ** -24 * np.abs(ref) + 2.0 ** -149)
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(got - ref) / ulp) < 4.0
    assert math.isclose(float(orc.swiglu(np.float32([1.0]), np.float32([1.0]))[0]),
                        1.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-6)


def test_swiglu_float32_order(orc):
    """Inputs on which the float32 operation order and a float64 evaluation rounded once differ."""
    # expf(100) overflows float32, so the float32 order gives a signed zero; in float64 the value
    # is about -3.7e-42, a float32 subnormal
    h = orc.swiglu(np.float32([-100.0, -100.0, -95.0]), np.float32([1.0, -1.0, 2.0]))
    assert h[0] == 0.0 and np.signbit(h[0])
    assert h[1] == 0.0 and not np.signbit(h[1])
    assert h[2] == 0.0 and np.signbit(h[2])
    dbl = np.float32(-100.0 / (1.0 + math.exp(100.0)))
    assert dbl != 0.0
    # finite range: each step rounded to float32, the exponential from float64 exp rounded once
    # (kept to arguments whose exponential is not within a tenth of an ulp of a rounding tie,
    # where libm's expf could round the other way)
    rng = np.random.default_rng(11)
    g = (rng.standard_normal(4000) * 3).astype(np.float32)
    u = rng.standard_normal(4000).astype(np.float32)
    ed = np.exp(-g.astype(np.float64))
    e32 = ed.astype(np.float32)
    frac = np.abs(ed - e32.astype(np.float64)) / np.spacing(np.abs(e32)).astype(np.float64)
    safe = np.abs(frac - 0.5) > 0.1
    den = np.float32(1.0) + e32
    step = (g / den) * u
    once = ((g.astype(np.float64) / (1.0 + ed)) * u.astype(np.float64)).astype(np.float32)
    pick = safe & (step != once)
    assert pick.sum() > 200
    got = orc.swiglu(g[pick], u[pick])
    assert np.array_equal(got, step[pick])
    assert not np.any(got == once[pick])


def _small_layer(key=0, fmt_gu=Q8_0, fmt_dn=Q8_0, n_embd=256, n_ff=128, E=8, T=1, k=2):
    import oracle
    tb = oracle.Tables(synth.nl4_table(key), synth.cb2_grid(key), synth.cb3_grid(key))
    gate, up, down = synth.experts(fmt_gu, fmt_dn, E, n_embd, n_ff, key)
    x = synth.activations(T, n_embd, key)
    lg = synth.router_logits(T, E, key)
    return tb, gate, up, down, x, lg


@pytest.mark.parametrize("fmts", [(Q8_0, Q8_0), (NL4, NL4), (CB3, Q8_0), (CB2, NL4)])
def test_layer_brute_force(orc, fmts):
    fg, fd = fmts
    n_embd, n_ff, E, T, k = (256, 256, 8, 3, 2) if fg in (CB2, CB3) else (256, 128, 8, 3, 2)
    tb, gate, up, down, x, lg = _small_layer(1, fg, fd, n_embd, n_ff, E, T, k)
    ids, w = orc.route_topk(lg, k)
    dst = np.array([5, 0, 3], np.int32)[:T]
    plan = orc.build_plan(ids, w.astype(np.float32), dst, E, 4)
    Y0 = synth.rng(3).standard_normal((6, n_embd)).astype(np.float32)
    res = orc.layer(x, plan, fg, fd, gate, up, down, n_embd, n_ff, Y0, tb)
    # dense float64 reference, token by token (no grouping), from the same quantized values
    Y = Y0.astype(np.float64).copy()
    for t in range(T):
        xd = np_dequant_q8_1(orc.quantize_q8_1(x[t]), n_embd)
        for j in range(k):
            e = ids[t, j]
            G = np_dequant(fg, gate[e], n_ff, n_embd, tb.nl4, tb.cb2, tb.cb3)
            U = np_dequant(fg, up[e], n_ff, n_embd, tb.nl4, tb.cb2, tb.cb3)
            g, u = G @ xd, U @ xd
            a = [a for a in res["gu"] if plan["ent_src"][a - 4] == t and
                 plan["grp_expert"][np.searchsorted(plan["grp_start"], a, "right") - 1] == e][0]
            assert np.allclose(res["gu"][a][0], g, rtol=0, atol=1e-12 * res["gu"][a][1].max())
            assert np.allclose(res["gu"][a][2], u, rtol=0, atol=1e-12 * res["gu"][a][3].max())
            hq = res["hq"][a]
            D = np_dequant(fd, down[e], n_embd, n_ff, tb.nl4, tb.cb2, tb.cb3)
            Y[dst[t]] += np.float32(w[t, j]) * (D @ np_dequant_q8_1(hq, n_ff))
    assert np.all(np.abs(res["Y"] - Y) <= 1e-12 * res["S"])
    untouched = [r for r in range(6) if r not in dst.tolist()]
    assert np.array_equal(res["Y"][untouched], Y0[untouched].astype(np.float64))


def test_two_calls_split_plan(orc):
    """Two calls of one layer over disjoint expert subsets, the second's entries past the first's
    ("#363 experts: ...", "Exactness": a call covers only its own entries, which may start past
    entry 0; both calls add into the same output rows), give the one-call result."""
    n_embd, n_ff, E, T, k = 256, 128, 8, 3, 2
    tb, gate, up, down, x, lg = _small_layer(2, Q8_0, Q8_0, n_embd, n_ff, E, T, k)
    ids, w = orc.route_topk(lg, k)
    dst = np.array([1, 4, 2], np.int32)
    plan = orc.build_plan(ids, w.astype(np.float32), dst, E, 4)
    pa, pb = synth.split_plan(plan, lambda e: e % 2 == 0)
    assert pa["n_groups"] + pb["n_groups"] == plan["n_groups"] and pa["n_groups"] and pb["n_groups"]
    assert pa["entry_base"] == 4 and pb["entry_base"] == pa["grp_start"][-1] == pb["grp_start"][0]
    assert pb["grp_start"][-1] == plan["grp_start"][-1]
    for p, par in ((pa, 0), (pb, 1)):
        assert np.all(np.diff(p["grp_expert"]) > 0) and np.all(p["grp_expert"] % 2 == par)
    # the same (expert, token, destination, weight) entries, each once
    def triples(p):
        out = []
        for g in range(p["n_groups"]):
            for a in range(p["grp_start"][g], p["grp_start"][g + 1]):
                r = a - p["entry_base"]
                out.append((int(p["grp_expert"][g]), int(p["ent_src"][r]), int(p["ent_dst"][r]),
                            float(p["ent_w"][r])))
        return sorted(out)
    assert triples(plan) == sorted(triples(pa) + triples(pb))
    Y0 = synth.rng(5).standard_normal((6, n_embd)).astype(np.float32)
    one = orc.layer(x, plan, Q8_0, Q8_0, gate, up, down, n_embd, n_ff, Y0, tb)
    ra = orc.layer(x, pa, Q8_0, Q8_0, gate, up, down, n_embd, n_ff, Y0, tb)
    rb = orc.layer(x, pb, Q8_0, Q8_0, gate, up, down, n_embd, n_ff, ra["Y"], tb)
    assert np.all(np.abs(rb["Y"] - one["Y"]) <= 1e-12 * one["S"])
    untouched = [r for r in range(6) if r not in dst.tolist()]
    assert np.array_equal(rb["Y"][untouched], Y0[untouched].astype(np.float64))
