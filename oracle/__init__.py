"""CPU oracle for the grouped routed-expert MoE decode step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
this package. It shares no code with the HIP library (``moe_routed_expert_route_amd``) and never
imports it. The arithmetic lives in ``oracle.c`` (plain C11, libm only); this module builds it with
gcc, binds it with ctypes and writes the per-entry layer loop out in the order the method states
it.

What it computes, from the pages this method is described on:

* "#363 experts: smaller and fewer launches for the verify window's PCIe call", opening paragraph
  and "What changes": a call runs the grouped gate/up, then SwiGLU and the q8_1 quantization over
  its own entries ``grp_start[0] .. grp_start[n_groups]``, then the grouped down; the SwiGLU
  product is a float32 value (rounded on its own) before it is quantized; "Exactness": entries
  may start past 0 and destinations may be scattered; rows a call does not own are not written.
* "#2058 Verify window: the routed experts' gate/up with the group's q8_1 rows in shared memory",
  "Why" and "Bit for bit": entries are grouped by expert so each expert's weights are decoded
  once; the entries of a group are independent, so the plain per-entry loop below *is* the
  result (grouping only changes which lane computes what).
* "#3455 GP100 (sm_60): 4-bit slots ...", "Validation": gate, up, h, hq and the combined output
  are compared stage by stage.

The per-entry output is scatter-added into its destination row with the entry's router weight,
in double, starting from the row's previous contents (readings listed in the design notes).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

Q8_0, NL4, CB2, CB3, Q5_1, NL4X = 1, 2, 3, 4, 5, 6
_BLOCK_BYTES = {Q8_0: 34, NL4: 18, CB2: 70, CB3: 110, Q5_1: 24, NL4X: 136}
_BLOCK_W = {Q8_0: 32, NL4: 32, CB2: 256, CB3: 256, Q5_1: 32, NL4X: 256}
_HEAD = {Q8_0: 2, NL4: 2, CB2: 2, CB3: 2, Q5_1: 4, NL4X: 8}   # block bytes before the codes

_P = ctypes.c_void_p
_I = ctypes.c_int


def build() -> str:
    """Compile oracle.c with gcc into liboracle.so (always recompiles)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_h2f.restype = ctypes.c_float
        L.orc_h2f.argtypes = [ctypes.c_uint16]
        L.orc_f2h.restype = ctypes.c_uint16
        L.orc_f2h.argtypes = [ctypes.c_float]
        L.orc_block_bytes.argtypes = [_I]
        L.orc_block_weights.argtypes = [_I]
        L.orc_quantize_q8_1.argtypes = [_P, _I, _P]
        L.orc_quantize_q8_0.argtypes = [_P, _I, _P]
        L.orc_decode_row.argtypes = [_I, _P, _I, _P, _P, _P, _P, _P, _P]
        L.orc_matvec.argtypes = [_I, _P, _I, _I, _P, _P, _P, _P, _P, _P]
        L.orc_swiglu.argtypes = [_P, _P, _I, _P]
        L.orc_route_topk.argtypes = [_P, _I, _I, _I, _P, _P]
        L.orc_build_plan.argtypes = [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class Tables:
    """The per-format lookup tables (NL4 16-entry int8 table, CB2 256x8 grid, CB3 512x4 grid)."""

    def __init__(self, nl4=None, cb2=None, cb3=None):
        self.nl4 = _c(nl4 if nl4 is not None else np.zeros(16), np.int8)
        self.cb2 = _c(cb2 if cb2 is not None else np.zeros(256 * 8), np.uint8)
        self.cb3 = _c(cb3 if cb3 is not None else np.zeros(512 * 4), np.uint8)

    def ptrs(self):
        return _ptr(self.nl4), _ptr(self.cb2), _ptr(self.cb3)


# ------------------------------------------------------------------ scalar helpers ------------

def h2f(h: int) -> float:
    return float(lib().orc_h2f(int(h)))


def f2h(f: float) -> int:
    return int(lib().orc_f2h(float(np.float32(f))))


def row_bytes(fmt: int, ncols: int) -> int:
    return ncols // _BLOCK_W[fmt] * _BLOCK_BYTES[fmt]


# ------------------------------------------------------------------ quantizers ----------------

def repack(fmt: int, mat, rows: int, ncols: int, to_planar: bool = True) -> np.ndarray:
    """The planar layout of a weight matrix, or back ("#3455 [Engine] GP100 (sm_60): 4-bit slots
    ...", "Approach": a load-time rewrite of the resident blocks that the decode reads, rebuilt and
    compared byte for byte). Per row: the row-major row is its blocks one after another; each block
    is its fp16 scale (2 bytes), its code bytes, and for CB2 / CB3 the 4 sub-scale bytes at its end.
    The planar row is every block's code bytes in block order, then every block's scale bytes (the
    header: fp16 scale, for Q5_1 also the fp16 offset; then for CB2 / CB3 the sub-scale bytes) in
    block order. Same bytes, same size."""
    B, W, H = _BLOCK_BYTES[fmt], _BLOCK_W[fmt], _HEAD[fmt]
    tail = 4 if fmt in (CB2, CB3) else 0   # sub-scale bytes at the end of a block
    nb = ncols // W
    m = np.asarray(mat, np.uint8).reshape(rows, nb * B)
    out = np.empty_like(m)
    ncode = B - H - tail
    for r in range(rows):
        if to_planar:
            blocks = m[r].reshape(nb, B)
            codes = blocks[:, H:H + ncode]
            scales = np.concatenate([blocks[:, :H], blocks[:, H + ncode:]], axis=1)
            out[r] = np.concatenate([codes.reshape(-1), scales.reshape(-1)])
        else:
            codes = m[r, :nb * ncode].reshape(nb, ncode)
            scales = m[r, nb * ncode:].reshape(nb, H + tail)
            out[r] = np.concatenate([scales[:, :H], codes, scales[:, H:]], axis=1).reshape(-1)
    return out.reshape(-1)


def quantize_q8_1(x) -> np.ndarray:
    """q8_1 blocks of the last axis (length a multiple of 32); returns uint8 [..., n/32*36]."""
    x = _c(x, np.float32)
    n = x.shape[-1]
    assert n % 32 == 0
    flat = x.reshape(-1, n)
    out = np.empty((flat.shape[0], n // 32 * 36), np.uint8)
    for r in range(flat.shape[0]):
        xr = np.ascontiguousarray(flat[r])
        lib().orc_quantize_q8_1(_ptr(xr), n, out[r].ctypes.data)
    return out.reshape(x.shape[:-1] + (n // 32 * 36,))


def quantize_q8_0(x) -> np.ndarray:
    x = _c(x, np.float32)
    n = x.shape[-1]
    assert n % 32 == 0
    flat = x.reshape(-1, n)
    out = np.empty((flat.shape[0], n // 32 * 34), np.uint8)
    for r in range(flat.shape[0]):
        xr = np.ascontiguousarray(flat[r])
        lib().orc_quantize_q8_0(_ptr(xr), n, out[r].ctypes.data)
    return out.reshape(x.shape[:-1] + (n // 32 * 34,))


# ------------------------------------------------------------------ decoders ------------------

def decode_row_offsets(fmt: int, row, ncols: int, tables: Tables):
    """(codes int32 [ncols], scales float64 [ncols/32], offsets float64 [ncols/32]) of one weight
    row: weight j = scales[j // 32] * codes[j] + offsets[j // 32] (offsets are 0 but for Q5_1)."""
    row = _c(row, np.uint8)
    codes = np.empty(ncols, np.int32)
    scales = np.empty(ncols // 32, np.float64)
    offsets = np.empty(ncols // 32, np.float64)
    rc = lib().orc_decode_row(fmt, _ptr(row), ncols, *tables.ptrs(), _ptr(codes), _ptr(scales),
                              _ptr(offsets))
    if rc != 0:
        raise ValueError("bad format or shape")
    return codes, scales, offsets


def decode_row(fmt: int, row, ncols: int, tables: Tables):
    """(codes int32 [ncols], scales float64 [ncols/32]) of one weight row."""
    codes, scales, _ = decode_row_offsets(fmt, row, ncols, tables)
    return codes, scales


def dequantize(fmt: int, mat, rows: int, ncols: int, tables: Tables) -> np.ndarray:
    """float64 [rows, ncols] weight values (scale * code + offset) of a row-major block matrix."""
    mat = _c(mat, np.uint8).reshape(rows, row_bytes(fmt, ncols))
    out = np.empty((rows, ncols), np.float64)
    for r in range(rows):
        codes, scales, offsets = decode_row_offsets(fmt, mat[r], ncols, tables)
        out[r] = codes.astype(np.float64) * np.repeat(scales, 32) + np.repeat(offsets, 32)
    return out


def matvec(fmt: int, mat, rows: int, ncols: int, xq, tables: Tables):
    """(out float64 [rows], S float64 [rows]): out[r] = sum_b c_b, S[r] = sum_b |c_b|."""
    mat = _c(mat, np.uint8)
    xq = _c(xq, np.uint8)
    assert mat.size >= rows * row_bytes(fmt, ncols) and xq.size >= ncols // 32 * 36
    out = np.empty(rows, np.float64)
    S = np.empty(rows, np.float64)
    rc = lib().orc_matvec(fmt, _ptr(mat), rows, ncols, _ptr(xq), *tables.ptrs(), _ptr(out), _ptr(S))
    if rc != 0:
        raise ValueError("bad format or shape")
    return out, S


def swiglu(g, u) -> np.ndarray:
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    h = np.empty_like(g)
    lib().orc_swiglu(_ptr(g), _ptr(u), g.size, _ptr(h))
    return h


# ------------------------------------------------------------------ routing / plan ------------

def route_topk(logits, k: int):
    """(ids int32 [T,k], w float64 [T,k])."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib().orc_route_topk(_ptr(logits), T, E, k, _ptr(ids), _ptr(w))
    return ids, w


def build_plan(ids, w, dst_of_token, E: int, entry_base: int = 0) -> dict:
    ids = _c(ids, np.int32)
    T, k = ids.shape
    w = None if w is None else _c(w, np.float32)
    dst = None if dst_of_token is None else _c(dst_of_token, np.int32)
    n = T * k
    grp_expert = np.zeros(max(n, 1), np.int32)
    grp_start = np.zeros(max(n, 1) + 1, np.int32)
    ent_src = np.zeros(max(n, 1), np.int32)
    ent_dst = np.zeros(max(n, 1), np.int32)
    ent_w = np.zeros(max(n, 1), np.float32)
    ng = lib().orc_build_plan(_ptr(ids), _ptr(w), _ptr(dst), T, k, E, entry_base, _ptr(grp_expert),
                              _ptr(grp_start), _ptr(ent_src), _ptr(ent_dst), _ptr(ent_w))
    if ng < 0:
        raise ValueError("expert id out of range")
    return dict(n_groups=ng, grp_expert=grp_expert[:ng].copy(), grp_start=grp_start[:ng + 1].copy(),
                entry_base=entry_base, ent_src=ent_src[:n].copy(), ent_dst=ent_dst[:n].copy(),
                ent_w=ent_w[:n].copy())


# ------------------------------------------------------------------ layer, stage by stage -----
# A plan here is a dict with n_groups, grp_expert[n_groups], grp_start[n_groups+1] (absolute
# entry indices) and ent_src / ent_dst / ent_w indexed by (absolute entry - entry_base).

def _entries(plan):
    base = int(plan["entry_base"])
    for g in range(int(plan["n_groups"])):
        e = int(plan["grp_expert"][g])
        for a in range(int(plan["grp_start"][g]), int(plan["grp_start"][g + 1])):
            yield g, e, a, a - base


def gate_up(plan, fmt, gate, up, n_embd, n_ff, xq_of_token, tables):
    """Per entry a (absolute index): g[a], u[a] = block dots of expert rows with xq[ent_src[a]].

    Returns dict absolute entry -> (g, Sg, u, Su), each float64 [n_ff]."""
    res = {}
    for _, e, a, r in _entries(plan):
        xq = xq_of_token[int(plan["ent_src"][r])]
        g, Sg = matvec(fmt, gate[e], n_ff, n_embd, xq, tables)
        u, Su = matvec(fmt, up[e], n_ff, n_embd, xq, tables)
        res[a] = (g, Sg, u, Su)
    return res


def down(plan, fmt, down_w, n_embd, n_ff, hq_of_entry, tables):
    """Per entry a: o[a] = block dots of the expert's down rows with hq[a]; dict a -> (o, So)."""
    res = {}
    for _, e, a, _r in _entries(plan):
        o, So = matvec(fmt, down_w[e], n_embd, n_ff, hq_of_entry[a], tables)
        res[a] = (o, So)
    return res


def scatter(plan, Y0, o_of_entry):
    """Y[dst] = Y0[dst] + sum over the call's entries of w * o (float64); rows no entry names keep
    Y0. Returns (Y float64, S float64) with S = |Y0| + sum |w| * So on written rows."""
    Y = np.array(Y0, dtype=np.float64, copy=True)
    S = np.abs(Y)
    for _, _, a, r in _entries(plan):
        d = int(plan["ent_dst"][r])
        w = float(plan["ent_w"][r])
        o, So = o_of_entry[a]
        Y[d] += w * o
        S[d] += abs(w) * So
    return Y, S


def layer(x, plan, fmt_gu, fmt_down, gate, up, down_w, n_embd, n_ff, Y0, tables):
    """The whole chain on the oracle's own values: x -> xq -> g,u -> h (float32) -> hq -> Y.

    Returns dict with xq, g/u (per entry), h, hq (per entry), Y, S."""
    x = _c(x, np.float32)
    xq = quantize_q8_1(x)
    gu = gate_up(plan, fmt_gu, gate, up, n_embd, n_ff, xq, tables)
    h, hq = {}, {}
    for a, (g, _, u, _) in gu.items():
        h[a] = swiglu(g.astype(np.float32), u.astype(np.float32))
        hq[a] = quantize_q8_1(h[a])
    o = down(plan, fmt_down, down_w, n_embd, n_ff, hq, tables)
    Y, S = scatter(plan, Y0, o)
    return dict(xq=xq, gu=gu, h=h, hq=hq, o=o, Y=Y, S=S)
