"""Seeded synthetic inputs for the grouped routed-expert decode step.

This module only draws random numbers and lays them out as bytes. It holds none of the method's
arithmetic (no quantization, decoding, routing, grouping or dot products): the tests, the oracle
and the GPU path all take their inputs from here, so a mistake in the method cannot hide in it.

Byte layouts follow the format readings (fp16 scale first): Q8_0 34 B / 32 weights, NL4 18 B /
32, CB2 70 B / 256, CB3 110 B / 256. Every draw is keyed: ``default_rng([BASE_SEED, *key])``.

Workload shapes (from the pages): 2560 x 768 expert matrices ("#363 ...", "Measured"), n_embd
2560 with n_ff 640 ("#2058 ...", "What changed"), windows of T = 1..4 tokens with top-8 experts
("#363 ...": cap_groups = window tokens x top-k).
"""
from __future__ import annotations

import numpy as np

BASE_SEED = 20261202

Q8_0, NL4, CB2, CB3, Q5_1, NL4X = 1, 2, 3, 4, 5, 6
FMT_NAMES = {"q8_0": Q8_0, "nl4": NL4, "cb2": CB2, "cb3": CB3}
BLOCK_BYTES = {Q8_0: 34, NL4: 18, CB2: 70, CB3: 110, Q5_1: 24, NL4X: 136}
BLOCK_WEIGHTS = {Q8_0: 32, NL4: 32, CB2: 256, CB3: 256, Q5_1: 32, NL4X: 256}

NAN_FILL = np.uint32(0x7FC0DEAD)   # quiet-NaN pattern put in rows a call must not write


def rng(*key) -> np.random.Generator:
    return np.random.default_rng([BASE_SEED, *[int(k) for k in key]])


def row_bytes(fmt: int, ncols: int) -> int:
    assert ncols % BLOCK_WEIGHTS[fmt] == 0, (fmt, ncols)
    return ncols // BLOCK_WEIGHTS[fmt] * BLOCK_BYTES[fmt]


# ------------------------------------------------------------------ tables --------------------

def nl4_table(*key) -> np.ndarray:
    """16 distinct int8 values drawn from U{-127..127}, sorted ascending."""
    v = rng(1, *key).choice(255, size=16, replace=False).astype(np.int64) - 127
    return np.sort(v).astype(np.int8)


def cb2_grid(*key) -> np.ndarray:
    """256 x 8 magnitudes in {1, 3, 5, 7} (uint8, row-major)."""
    return (2 * rng(2, *key).integers(0, 4, size=256 * 8) + 1).astype(np.uint8)


def cb3_grid(*key) -> np.ndarray:
    """512 x 4 magnitudes in {1, 3, ..., 15} (uint8, row-major)."""
    return (2 * rng(3, *key).integers(0, 8, size=512 * 4) + 1).astype(np.uint8)


# ------------------------------------------------------------------ weights -------------------

def fp16_scales(g: np.random.Generator, n: int, lo: float = 1e-3, hi: float = 1e-2) -> np.ndarray:
    """n fp16 scales drawn from U[lo, hi], as raw uint16 bit patterns."""
    return g.uniform(lo, hi, size=n).astype(np.float16).view(np.uint16)


def weight_matrix(fmt: int, rows: int, cols: int, *key) -> np.ndarray:
    """Bytes of a rows x cols weight matrix in `fmt`, row-major blocks (uint8 [rows*row_bytes]).

    Codes are uniform over every bit pattern the format allows (Q8_0 quants U{-127..127});
    the fp16 scale of each block is U[1e-3, 1e-2] (NL4X: U[1e-4, 1e-3], times its 6-bit sub-block
    scale minus 32); a Q5_1 block's fp16 offset is about -15.5 scales (times U[0.9, 1.1]), so its
    32 code levels straddle zero."""
    g = rng(10, fmt, rows, cols, *key)
    bsz = BLOCK_BYTES[fmt]
    nblk = rows * cols // BLOCK_WEIGHTS[fmt]
    blocks = g.integers(0, 256, size=(nblk, bsz), dtype=np.uint8)
    if fmt == Q8_0:
        blocks[:, 2:] = g.integers(-127, 128, size=(nblk, 32), dtype=np.int8).view(np.uint8)
    # NL4X: the super-block scale is multiplied by l - 32 (|l - 32| about 16 on average), so it is
    # drawn ten times smaller to keep the weights' magnitudes those of the other formats
    sc = fp16_scales(g, nblk, 1e-4, 1e-3) if fmt == NL4X else fp16_scales(g, nblk)
    blocks[:, 0] = (sc & 0xFF).astype(np.uint8)
    blocks[:, 1] = (sc >> 8).astype(np.uint8)
    if fmt == Q5_1:
        d = sc.astype(np.uint16).view(np.float16).astype(np.float64)
        m = (-15.5 * d * g.uniform(0.9, 1.1, size=nblk)).astype(np.float16).view(np.uint16)
        blocks[:, 2] = (m & 0xFF).astype(np.uint8)
        blocks[:, 3] = (m >> 8).astype(np.uint8)
    return blocks.reshape(-1)


def experts(fmt_gu: int, fmt_down: int, n_experts: int, n_embd: int, n_ff: int, *key):
    """Lists gate[e], up[e] (n_ff x n_embd) and down[e] (n_embd x n_ff) of byte arrays."""
    gate = [weight_matrix(fmt_gu, n_ff, n_embd, *key, e, 0) for e in range(n_experts)]
    up = [weight_matrix(fmt_gu, n_ff, n_embd, *key, e, 1) for e in range(n_experts)]
    down = [weight_matrix(fmt_down, n_embd, n_ff, *key, e, 2) for e in range(n_experts)]
    return gate, up, down


# ------------------------------------------------------------------ activations / routing -----

def activations(T: int, n: int, *key) -> np.ndarray:
    """x float32 [T, n] ~ N(0, 1)."""
    return rng(20, *key).standard_normal((T, n)).astype(np.float32)


def router_logits(T: int, E: int, *key) -> np.ndarray:
    """Router logits float32 [T, E] ~ N(0, 1)."""
    return rng(21, *key).standard_normal((T, E)).astype(np.float32)


def zipf_ids(T: int, E: int, k: int, s: float, *key) -> np.ndarray:
    """Per token, k distinct experts drawn one after another without replacement with
    P(rank r) proportional to r^-s; rank -> expert through a seeded permutation."""
    g = rng(22, *key)
    perm = g.permutation(E)
    base = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        p = base.copy()
        for j in range(k):
            r = g.choice(E, p=p / p.sum())
            ids[t, j] = perm[r]
            p[r] = 0.0
    return ids


def uniform_ids(T: int, E: int, k: int, *key) -> np.ndarray:
    g = rng(23, *key)
    return np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)


def shared_ids(T: int, E: int, k: int, *key) -> np.ndarray:
    """All T tokens route to the same k experts (k groups of T entries each)."""
    g = rng(24, *key)
    one = g.choice(E, size=k, replace=False).astype(np.int32)
    return np.tile(one, (T, 1))


def logits_for_ids(ids: np.ndarray, E: int, *key) -> np.ndarray:
    """Router logits float32 [T, E] whose top-k experts are exactly `ids` [T, k]: the chosen
    experts get N(0, 1) logits, every other expert N(0, 1) - 20 (so ranks are never tied)."""
    ids = np.asarray(ids)
    T, k = ids.shape
    g = rng(25, *key)
    lg = (g.standard_normal((T, E)) - 20.0).astype(np.float32)
    for t in range(T):
        lg[t, ids[t]] = g.standard_normal(k).astype(np.float32)
    return lg


def direct_plan(n_groups: int, E: int, T: int, n_rows: int, entry_base: int, *key,
                max_entries: int | None = None) -> dict:
    """A plan built directly (no routing): n_groups distinct experts ascending, 1..T entries per
    group with distinct tokens ascending (at most max_entries in all), tokens mapped to scattered
    destination rows of an n_rows-row output, router weights U(0.05, 1). Entry indices start at
    entry_base."""
    g = rng(26, n_groups, *key)
    exps = np.sort(g.choice(E, size=n_groups, replace=False)).astype(np.int32) if n_groups else \
        np.zeros(0, np.int32)
    dst_of_token = g.choice(n_rows, size=T, replace=False).astype(np.int32)
    counts = g.integers(1, T + 1, size=n_groups) if n_groups else np.zeros(0, np.int64)
    if max_entries is not None:
        assert n_groups <= max_entries
        while counts.sum() > max_entries:
            big = np.flatnonzero(counts > 1)
            counts[big[g.integers(len(big))]] -= 1
    src, starts = [], [entry_base]
    for c in counts:
        src.extend(np.sort(g.choice(T, size=int(c), replace=False)).tolist())
        starts.append(starts[-1] + int(c))
    src = np.asarray(src, np.int32)
    return dict(n_groups=int(n_groups), grp_expert=exps, grp_start=np.asarray(starts, np.int32),
                entry_base=int(entry_base), ent_src=src, ent_dst=dst_of_token[src].astype(np.int32),
                ent_w=g.uniform(0.05, 1.0, size=len(src)).astype(np.float32), T=T)


def split_plan(plan: dict, first) -> tuple[dict, dict]:
    """Two calls' plans from one: the groups whose expert satisfies first(e) go to the first call,
    the rest to the second, each keeping its groups ascending by expert. The entries are laid out
    again in one shared run of entry indices starting at plan["entry_base"]: the first call's
    entries, then the second's, so the second call starts past the first's entries. Entry order
    inside a group is kept."""
    ng, base = int(plan["n_groups"]), int(plan["entry_base"])
    gs = np.asarray(plan["grp_start"], np.int64)
    parts = ([], [])
    for g in range(ng):
        parts[0 if first(int(plan["grp_expert"][g])) else 1].append(g)
    out, at = [], base
    for gl in parts:
        starts, rows = [at], []
        for g in gl:
            rows.extend(range(int(gs[g]) - base, int(gs[g + 1]) - base))
            starts.append(starts[-1] + int(gs[g + 1] - gs[g]))
        rows = np.asarray(rows, np.int64)
        out.append(dict(n_groups=len(gl), grp_expert=np.asarray([plan["grp_expert"][g] for g in gl], np.int32),
                        grp_start=np.asarray(starts, np.int32), entry_base=at,
                        ent_src=np.asarray(plan["ent_src"], np.int32)[rows],
                        ent_dst=np.asarray(plan["ent_dst"], np.int32)[rows],
                        ent_w=np.asarray(plan["ent_w"], np.float32)[rows]))
        at = starts[-1]
    return out[0], out[1]


def nan_rows(n_rows: int, n: int) -> np.ndarray:
    """float32 [n_rows, n] filled with the quiet-NaN pattern 0x7FC0DEAD."""
    return np.full((n_rows, n), NAN_FILL, np.uint32).view(np.float32)
