"""Python binding of libmoe_route.so: the C-ABI entry points under the same names.

Argument marshalling only: torch tensors supply device memory and the current HIP stream; every
step of the computation runs in the library's HIP kernels. If the library is not built the
functions raise (there is no fallback of any kind).
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_route.so")

Q8_0, NL4, CB2, CB3, Q5_1, NL4X = 1, 2, 3, 4, 5, 6
BLOCK_BYTES = {Q8_0: 34, NL4: 18, CB2: 70, CB3: 110, Q5_1: 24, NL4X: 136}
BLOCK_WEIGHTS = {Q8_0: 32, NL4: 32, CB2: 256, CB3: 256, Q5_1: 32, NL4X: 256}

ERR_BITS = {1: "NGROUPS", 2: "ENTRIES", 4: "EXPERT", 8: "SRC", 16: "DST", 32: "ALIGN", 64: "WAIT"}

EXPORTS = ("moe_route_topk", "moe_build_plan", "moe_quantize_q8_1", "moe_repack", "moe_gate_up",
           "moe_swiglu_q8_1", "moe_down_scatter", "moe_workspace_bytes",
           "moe_layer_decode", "moe_layer_decode_routed", "moe_layer_decode_routed_noalloc", "moe_layer_step", "moe_layer_gate_up",
           "moe_layer_down",
           "moe_workspace_layout", "moe_prefill_plan", "moe_prefill_gate_up", "moe_prefill_swiglu_q8_1",
           "moe_prefill_down", "moe_prefill_scatter",
           "moe_stream_read", "moe_status_string", "moe_last_error")

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int


class MoeLayer(ctypes.Structure):
    _fields_ = [("n_embd", ctypes.c_int32), ("n_ff", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("fmt_gate_up", ctypes.c_int32), ("fmt_down", ctypes.c_int32),
                ("gate", _P), ("up", _P), ("down", _P),
                ("nl4_table", _P), ("cb2_grid", _P), ("cb3_grid", _P)]


class MoePlan(ctypes.Structure):
    _fields_ = [("cap_groups", ctypes.c_int32), ("cap_entries", ctypes.c_int32),
                ("n_groups", _P), ("grp_expert", _P), ("grp_start", _P), ("ent_src", _P),
                ("ent_dst", _P), ("ent_w", _P), ("err", _P)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_route_topk.argtypes = [_P, _P, _I, _I, _I, _P, _P]
        L.moe_build_plan.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, ctypes.POINTER(MoePlan)]
        L.moe_quantize_q8_1.argtypes = [_P, _P, _I, _I, _P]
        L.moe_repack.argtypes = [_P, _I, _P, ctypes.c_int64, _I, _P, _I]
        L.moe_gate_up.argtypes = [_P, ctypes.POINTER(MoeLayer), ctypes.POINTER(MoePlan), _P, _I, _P,
                                  _P, _I, _I]
        L.moe_swiglu_q8_1.argtypes = [_P, ctypes.POINTER(MoePlan), _P, _P, _I, _I, _P, _P]
        L.moe_down_scatter.argtypes = [_P, ctypes.POINTER(MoeLayer), ctypes.POINTER(MoePlan), _P, _P,
                                       _I, _I, _I]
        L.moe_workspace_bytes.argtypes = [ctypes.POINTER(MoeLayer), ctypes.POINTER(MoePlan)]
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_layer_decode.argtypes = [_P, ctypes.POINTER(MoeLayer), ctypes.POINTER(MoePlan), _P, _I,
                                       _P, _I, _I, _P, ctypes.c_size_t, _I]
        L.moe_layer_decode_routed.argtypes = [_P, ctypes.POINTER(MoeLayer), ctypes.POINTER(MoePlan),
                                              _P, _I, _I, _P, _I, _P, _P, _I, _I, _P,
                                              ctypes.c_size_t, _I]
        L.moe_layer_decode_routed_noalloc.argtypes = [_P, ctypes.POINTER(MoeLayer), ctypes.POINTER(MoePlan),
                                                      _P, _I, _I, _P, _I, _P, _P, _I, _I, _I]
        L.moe_layer_step.argtypes = [_P, ctypes.POINTER(MoeLayer), ctypes.POINTER(MoePlan),
                                     _P, _I, _I, _P, _I, _P, _P, _I, _I, _P, ctypes.c_size_t, _I]
        L.moe_layer_gate_up.argtypes = [_P, ctypes.POINTER(MoeLayer), ctypes.POINTER(MoePlan), _P, _I,
                                        _I, _P, _I, _P, _I, _P, ctypes.c_size_t, _I]
        L.moe_layer_down.argtypes = [_P, ctypes.POINTER(MoeLayer), ctypes.POINTER(MoePlan), _P,
                                     ctypes.c_size_t, _I, _P, _I, _I, _I]
        L.moe_workspace_layout.argtypes = [ctypes.POINTER(MoeLayer), ctypes.POINTER(MoePlan), _P]
        L.moe_prefill_plan.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, ctypes.POINTER(MoePlan), _P]
        L.moe_prefill_gate_up.argtypes = [_P, ctypes.POINTER(MoeLayer), ctypes.POINTER(MoePlan), _P, _I, _P,
                                          _P, _I]
        L.moe_prefill_swiglu_q8_1.argtypes = [_P, ctypes.POINTER(MoePlan), _P, _P, _I, _I, _P, _P]
        L.moe_prefill_down.argtypes = [_P, ctypes.POINTER(MoeLayer), ctypes.POINTER(MoePlan), _P, _P, _I]
        L.moe_prefill_scatter.argtypes = [_P, ctypes.POINTER(MoePlan), _P, _P, _I, _I, _P, _I, _I, _P, _I, _I]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [_I]
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_stream_read.argtypes = [_P, _P, ctypes.c_uint64, _P, _I]
        _lib = L
    return _lib


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc: int, what: str):
    if rc != 0:
        L = lib()
        msg = L.moe_status_string(rc).decode()
        extra = L.moe_last_error().decode() if rc in (-4, -5) else ""
        raise RuntimeError(f"{what}: {msg} ({rc}) {extra}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# ------------------------------------------------------------------ device-side objects -------

class Layer:
    """One layer's experts on the device: byte tensors per expert, device pointer arrays and the
    C struct. `gate`, `up`, `down` are lists of uint8 tensors (or host arrays, uploaded)."""

    def __init__(self, n_embd, n_ff, fmt_gate_up, fmt_down, gate, up, down, nl4=None, cb2=None,
                 cb3=None, device="cuda"):
        def dev(a, dtype=torch.uint8):
            if a is None:
                return None
            t = a if isinstance(a, torch.Tensor) else torch.from_numpy(a)
            return t.to(device=device, dtype=dtype).contiguous()
        self.gate = [dev(a) for a in gate]
        self.up = [dev(a) for a in up]
        self.down = [dev(a) for a in down]
        self.nl4 = dev(nl4, torch.int8)
        self.cb2 = dev(cb2)
        self.cb3 = dev(cb3)
        self.ptr_gate = torch.tensor([t.data_ptr() for t in self.gate], dtype=torch.int64, device=device)
        self.ptr_up = torch.tensor([t.data_ptr() for t in self.up], dtype=torch.int64, device=device)
        self.ptr_down = torch.tensor([t.data_ptr() for t in self.down], dtype=torch.int64, device=device)
        self.n_embd, self.n_ff = n_embd, n_ff
        self.fmt_gate_up, self.fmt_down = fmt_gate_up, fmt_down
        self.struct = MoeLayer(n_embd, n_ff, len(self.gate), fmt_gate_up, fmt_down,
                               self.ptr_gate.data_ptr(), self.ptr_up.data_ptr(),
                               self.ptr_down.data_ptr(),
                               self.nl4.data_ptr() if self.nl4 is not None else None,
                               self.cb2.data_ptr() if self.cb2 is not None else None,
                               self.cb3.data_ptr() if self.cb3 is not None else None)

    @classmethod
    def from_pointers(cls, n_embd, n_ff, fmt_gate_up, fmt_down, ptr_gate, ptr_up, ptr_down,
                      nl4=None, cb2=None, cb3=None, keep=()):
        """Experts already resident elsewhere (e.g. a pool); ptr_* are int64 device tensors."""
        self = cls.__new__(cls)
        self.gate = self.up = self.down = []
        self.nl4, self.cb2, self.cb3 = nl4, cb2, cb3
        self.ptr_gate, self.ptr_up, self.ptr_down = ptr_gate, ptr_up, ptr_down
        self._keep = keep
        self.n_embd, self.n_ff = n_embd, n_ff
        self.fmt_gate_up, self.fmt_down = fmt_gate_up, fmt_down
        self.struct = MoeLayer(n_embd, n_ff, int(ptr_gate.numel()), fmt_gate_up, fmt_down,
                               ptr_gate.data_ptr(), ptr_up.data_ptr(), ptr_down.data_ptr(),
                               nl4.data_ptr() if nl4 is not None else None,
                               cb2.data_ptr() if cb2 is not None else None,
                               cb3.data_ptr() if cb3 is not None else None)
        return self


class Plan:
    """Device arrays of a call's plan. Entry arrays hold `entry_capacity` entries (absolute
    indices), so a plan may start past entry 0."""

    def __init__(self, cap_groups, cap_entries, entry_capacity=None, device="cuda", entries_of=None):
        """entries_of: another Plan whose entry arrays (and error word) this one shares, so that
        two calls of one layer (each over its own groups) index one run of entries."""
        ec = entry_capacity if entry_capacity is not None else cap_entries
        i32 = dict(dtype=torch.int32, device=device)
        self.n_groups = torch.zeros(1, **i32)
        self.grp_expert = torch.zeros(cap_groups, **i32)
        self.grp_start = torch.zeros(cap_groups + 1, **i32)
        if entries_of is not None:
            self.ent_src, self.ent_dst = entries_of.ent_src, entries_of.ent_dst
            self.ent_w, self.err = entries_of.ent_w, entries_of.err
        else:
            self.ent_src = torch.zeros(ec, **i32)
            self.ent_dst = torch.zeros(ec, **i32)
            self.ent_w = torch.zeros(ec, dtype=torch.float32, device=device)
            self.err = torch.zeros(1, **i32)
        self.cap_groups, self.cap_entries = cap_groups, cap_entries
        self.struct = MoePlan(cap_groups, cap_entries, self.n_groups.data_ptr(),
                              self.grp_expert.data_ptr(), self.grp_start.data_ptr(),
                              self.ent_src.data_ptr(), self.ent_dst.data_ptr(),
                              self.ent_w.data_ptr(), self.err.data_ptr())

    def set(self, plan: dict):
        """Copy a host plan (dict of numpy arrays with absolute entry indices) in."""
        ng = int(plan["n_groups"])
        base = int(plan["entry_base"])
        self.n_groups.fill_(ng)
        if ng:
            self.grp_expert[:ng].copy_(torch.as_tensor(plan["grp_expert"][:ng], dtype=torch.int32))
        self.grp_start[:ng + 1].copy_(torch.as_tensor(plan["grp_start"][:ng + 1], dtype=torch.int32))
        n = len(plan["ent_src"])
        if n:
            self.ent_src[base:base + n].copy_(torch.as_tensor(plan["ent_src"], dtype=torch.int32))
            self.ent_dst[base:base + n].copy_(torch.as_tensor(plan["ent_dst"], dtype=torch.int32))
            self.ent_w[base:base + n].copy_(torch.as_tensor(plan["ent_w"], dtype=torch.float32))

    def get(self) -> dict:
        """Host copy (synchronises)."""
        ng = int(self.n_groups.item())
        gs = self.grp_start[:ng + 1].cpu().numpy()
        base = int(gs[0]) if ng else 0
        end = int(gs[-1]) if ng else 0
        return dict(n_groups=ng, grp_expert=self.grp_expert[:ng].cpu().numpy(), grp_start=gs,
                    entry_base=base, ent_src=self.ent_src[base:end].cpu().numpy(),
                    ent_dst=self.ent_dst[base:end].cpu().numpy(),
                    ent_w=self.ent_w[base:end].cpu().numpy())

    def errors(self) -> int:
        return int(self.err.item()) & 0xFFFFFFFF


# ------------------------------------------------------------------ entry points --------------

LAYOUT_PLANAR = 0x100   # OR-ed into a layer's format field: planar rows (see moe_repack)


def moe_repack(fmt, src, rows, cols, dst=None, to_planar=True, stream=None):
    """rows x cols weights of base format `fmt` (uint8 device tensor `src`) into the planar layout
    (to_planar) or back into the row-major one; returns dst (a new tensor unless given)."""
    dst = dst if dst is not None else torch.empty_like(src)
    _check(lib().moe_repack(_stream(stream), int(fmt), _ptr(src), int(rows), int(cols), _ptr(dst),
                            1 if to_planar else 0), "moe_repack")
    return dst


# ------------------------------------------------------------------ prompt path ---------------

def moe_prefill_plan(ids, w, plan: Plan, E, dst_of_token=None, entry_base=0, ent_of=None, stream=None):
    """Plan of T x k choices (ids, w int32 / float32 [T, k] device tensors); returns ent_of [T, k]."""
    T, k = ids.shape
    ent_of = ent_of if ent_of is not None else torch.empty((T, k), dtype=torch.int32, device=ids.device)
    _check(lib().moe_prefill_plan(_stream(stream), _ptr(ids), _ptr(w), _ptr(dst_of_token), T, k, E,
                                  entry_base, ctypes.byref(plan.struct), _ptr(ent_of)), "moe_prefill_plan")
    return ent_of


def moe_prefill_gate_up(layer: Layer, plan: Plan, xq, g, u, stream=None):
    _check(lib().moe_prefill_gate_up(_stream(stream), ctypes.byref(layer.struct), ctypes.byref(plan.struct),
                                     _ptr(xq), xq.shape[0], _ptr(g), _ptr(u), g.stride(0)),
           "moe_prefill_gate_up")


def moe_prefill_swiglu_q8_1(plan: Plan, g, u, n_ff, hq, h=None, stream=None):
    _check(lib().moe_prefill_swiglu_q8_1(_stream(stream), ctypes.byref(plan.struct), _ptr(g), _ptr(u), n_ff,
                                         g.stride(0), _ptr(h), _ptr(hq)), "moe_prefill_swiglu_q8_1")


def moe_prefill_down(layer: Layer, plan: Plan, hq, O, stream=None):
    _check(lib().moe_prefill_down(_stream(stream), ctypes.byref(layer.struct), ctypes.byref(plan.struct),
                                  _ptr(hq), _ptr(O), O.stride(0)), "moe_prefill_down")


def moe_prefill_scatter(plan: Plan, ent_of, O, Y, n_embd, dst_of_token=None, stream=None):
    T, k = ent_of.shape
    _check(lib().moe_prefill_scatter(_stream(stream), ctypes.byref(plan.struct), _ptr(ent_of),
                                     _ptr(dst_of_token), T, k, _ptr(O), O.stride(0), n_embd, _ptr(Y),
                                     Y.shape[0], Y.stride(0)), "moe_prefill_scatter")


def moe_route_topk(logits, k, ids=None, w=None, stream=None):
    T, E = logits.shape
    ids = ids if ids is not None else torch.empty((T, k), dtype=torch.int32, device=logits.device)
    w = w if w is not None else torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(lib().moe_route_topk(_stream(stream), _ptr(logits), T, E, k, _ptr(ids), _ptr(w)),
           "moe_route_topk")
    return ids, w


def moe_build_plan(ids, w, plan: Plan, E, dst_of_token=None, entry_base=0, stream=None):
    T, k = ids.shape
    _check(lib().moe_build_plan(_stream(stream), _ptr(ids), _ptr(w), _ptr(dst_of_token), T, k, E,
                                entry_base, ctypes.byref(plan.struct)), "moe_build_plan")


def moe_quantize_q8_1(x, q=None, stream=None):
    rows, n = x.shape
    q = q if q is not None else torch.empty((rows, n // 32 * 36), dtype=torch.uint8, device=x.device)
    _check(lib().moe_quantize_q8_1(_stream(stream), _ptr(x), rows, n, _ptr(q)), "moe_quantize_q8_1")
    return q


def moe_gate_up(layer: Layer, plan: Plan, xq, g, u, grid_limit=0, stream=None):
    _check(lib().moe_gate_up(_stream(stream), ctypes.byref(layer.struct), ctypes.byref(plan.struct),
                             _ptr(xq), xq.shape[0], _ptr(g), _ptr(u), g.stride(0), grid_limit),
           "moe_gate_up")


def moe_swiglu_q8_1(plan: Plan, g, u, n_ff, hq, h=None, stream=None):
    _check(lib().moe_swiglu_q8_1(_stream(stream), ctypes.byref(plan.struct), _ptr(g), _ptr(u), n_ff,
                                 g.stride(0), _ptr(h), _ptr(hq)), "moe_swiglu_q8_1")


def moe_workspace_bytes(layer: Layer, plan: Plan) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(layer.struct), ctypes.byref(plan.struct)))


def workspace(layer: Layer, plan: Plan, device="cuda"):
    """Allocate a zero-filled workspace for this layer geometry and plan capacity (the one-launch
    step needs its flags and counts zero before the first call; every other call reads only bytes
    it wrote itself)."""
    nb = moe_workspace_bytes(layer, plan)
    if nb == 0:
        raise RuntimeError("moe_workspace_bytes: bad layer or plan")
    ws = torch.zeros(nb, dtype=torch.uint8, device=device)
    if ws.data_ptr() % 256:
        raise RuntimeError("workspace not 256-byte aligned")
    return ws


def moe_workspace_layout(layer: Layer, plan: Plan):
    """Byte offsets of the split q8_1 rows of h in the workspace: low quant halves, high quant
    halves, float scales."""
    off = (ctypes.c_size_t * 3)()
    _check(lib().moe_workspace_layout(ctypes.byref(layer.struct), ctypes.byref(plan.struct), off),
           "moe_workspace_layout")
    return [int(v) for v in off]


def moe_down_scatter(layer: Layer, plan: Plan, hq, Y, grid_limit=0, stream=None):
    _check(lib().moe_down_scatter(_stream(stream), ctypes.byref(layer.struct), ctypes.byref(plan.struct),
                                  _ptr(hq), _ptr(Y), Y.shape[0], Y.stride(0), grid_limit),
           "moe_down_scatter")


def moe_layer_decode(layer: Layer, plan: Plan, x, Y, ws, grid_limit=0, stream=None):
    _check(lib().moe_layer_decode(_stream(stream), ctypes.byref(layer.struct), ctypes.byref(plan.struct),
                                  _ptr(x), x.shape[0], _ptr(Y), Y.shape[0], Y.stride(0), _ptr(ws),
                                  ws.numel(), grid_limit), "moe_layer_decode")


def moe_layer_decode_routed(layer: Layer, plan: Plan, logits, k, x, Y, ws, dst_of_token=None,
                            entry_base=0, grid_limit=0, stream=None):
    T = logits.shape[0]
    _check(lib().moe_layer_decode_routed(_stream(stream), ctypes.byref(layer.struct),
                                         ctypes.byref(plan.struct), _ptr(logits), T, k,
                                         _ptr(dst_of_token), entry_base, _ptr(x), _ptr(Y), Y.shape[0],
                                         Y.stride(0), _ptr(ws), ws.numel(), grid_limit),
           "moe_layer_decode_routed")


def moe_layer_decode_routed_noalloc(layer: Layer, plan: Plan, logits, k, x, Y, dst_of_token=None,
                                    entry_base=0, grid_limit=0, stream=None):
    """moe_layer_decode_routed with the library's static scratch as its workspace (nothing is
    allocated); calls that overlap on one GPU race."""
    T = logits.shape[0]
    _check(lib().moe_layer_decode_routed_noalloc(_stream(stream), ctypes.byref(layer.struct),
                                                 ctypes.byref(plan.struct), _ptr(logits), T, k,
                                                 _ptr(dst_of_token), entry_base, _ptr(x), _ptr(Y), Y.shape[0],
                                                 Y.stride(0), grid_limit),
           "moe_layer_decode_routed_noalloc")


def moe_layer_step(layer: Layer, plan: Plan, logits, k, x, Y, ws, dst_of_token=None, entry_base=0,
                   grid_limit=0, stream=None):
    """The whole step from the logits in one launch (workgroups meet through counts in ws)."""
    T = logits.shape[0]
    _check(lib().moe_layer_step(_stream(stream), ctypes.byref(layer.struct), ctypes.byref(plan.struct),
                                _ptr(logits), T, k, _ptr(dst_of_token), entry_base, _ptr(x), _ptr(Y),
                                Y.shape[0], Y.stride(0), _ptr(ws), ws.numel(), grid_limit),
           "moe_layer_step")


def moe_layer_gate_up(layer: Layer, plan: Plan, x, ws, logits=None, k=0, dst_of_token=None,
                      entry_base=0, grid_limit=0, stream=None):
    """First launch of the layer step (routing and grouping too when logits are given)."""
    T = logits.shape[0] if logits is not None else 0
    _check(lib().moe_layer_gate_up(_stream(stream), ctypes.byref(layer.struct), ctypes.byref(plan.struct),
                                   _ptr(logits), T, k, _ptr(dst_of_token), entry_base, _ptr(x),
                                   x.shape[0], _ptr(ws), ws.numel(), grid_limit), "moe_layer_gate_up")


def moe_layer_down(layer: Layer, plan: Plan, ws, n_tokens, Y, grid_limit=0, stream=None):
    """Second launch of the layer step: down over the workspace's h rows + scatter into Y."""
    _check(lib().moe_layer_down(_stream(stream), ctypes.byref(layer.struct), ctypes.byref(plan.struct),
                                _ptr(ws), ws.numel(), n_tokens, _ptr(Y), Y.shape[0], Y.stride(0),
                                grid_limit), "moe_layer_down")


def moe_stream_read(buf, out, grid, stream=None):
    """The achievable-bandwidth reference: one streaming read of `buf` (a contiguous device tensor
    of a multiple of 16 bytes) by `grid` workgroups; out[b] (uint32 or int32, >= grid words) gets
    the XOR of the 32-bit words workgroup b read."""
    assert buf.is_contiguous() and out.numel() >= grid and out.element_size() == 4
    _check(lib().moe_stream_read(_stream(stream), _ptr(buf), buf.numel() * buf.element_size(), _ptr(out),
                                 grid), "moe_stream_read")
