"""The entry point that allocates nothing (moe_layer_decode_routed_noalloc: the workspace is the
library's static per-GPU scratch) against moe_layer_decode_routed with a caller's workspace,
through the C-ABI: the same plan and the same Y, bit for bit, on two calls in a row, the second
on a smaller layer (the scratch then holds the first call's bytes). An oversize layer is rejected
on the host before anything is enqueued (no GPU needed)."""
import ctypes

import numpy as np
import pytest
import torch

from moe_routed_expert_route_amd import binding as B

Q8_0, NL4 = 1, 2


def _run_pair(c, dst, base):
    d = torch.device("cuda:0")
    T, k = c.T, c.k
    lg = torch.from_numpy(c.logits).to(d)
    x = torch.from_numpy(c.x).to(d)
    n_rows = T + 3
    dt = torch.as_tensor(dst, dtype=torch.int32, device=d)
    from . import gpu_util as U
    Y0 = U.y0_for(n_rows, c.n_embd, dst, 9)
    out = []
    for noalloc in (False, True):
        plan = B.Plan(T * k, T * k, entry_capacity=base + T * k, device=d)
        Y = torch.from_numpy(Y0.copy()).to(d)
        if noalloc:
            B.moe_layer_decode_routed_noalloc(c.layer, plan, lg, k, x, Y, dst_of_token=dt, entry_base=base)
        else:
            ws = B.workspace(c.layer, plan, device=d)
            B.moe_layer_decode_routed(c.layer, plan, lg, k, x, Y, ws, dst_of_token=dt, entry_base=base)
        torch.cuda.synchronize()
        assert plan.errors() == 0
        out.append((plan.get(), Y.cpu().numpy()))
    (pa, ya), (pb, yb) = out
    for key in ("n_groups", "grp_expert", "grp_start", "ent_src", "ent_dst"):
        assert np.array_equal(np.asarray(pa[key]), np.asarray(pb[key])), key
    assert np.array_equal(U.bits(pa["ent_w"]), U.bits(pb["ent_w"]))
    assert np.array_equal(U.bits(ya), U.bits(yb))
    return ya


@pytest.mark.gpu
def test_noalloc_two_calls_match_workspace_path():
    from . import gpu_util as U
    big = U.routed_case("noalloc_big", 2560, 768, 128, 8, 4, NL4, NL4, 31)
    Y = _run_pair(big, np.array([2, 5, 0, 6], np.int32), 3)
    assert np.isfinite(Y[[0, 2, 5, 6]]).all()
    small = U.routed_case("noalloc_small", 256, 128, 8, 2, 1, Q8_0, Q8_0, 32)
    _run_pair(small, np.array([1], np.int32), 0)


def test_noalloc_rejects_oversize_on_host():
    import os
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("library not built")
    L = B.lib()
    fake = ctypes.c_void_p(256)
    layer = B.MoeLayer(2560, 8192, 8, Q8_0, Q8_0, fake, fake, fake, None, None, None)
    plan = B.MoePlan(64, 64, fake, fake, fake, fake, fake, fake, fake)
    need = L.moe_workspace_bytes(ctypes.byref(layer), ctypes.byref(plan))
    assert need > (512 << 10)
    rc = L.moe_layer_decode_routed_noalloc(None, ctypes.byref(layer), ctypes.byref(plan), fake, 8, 8, None, 0,
                                           fake, fake, 8, 2560, 0)
    assert rc == -5                                            # MOE_E_WS, nothing enqueued
    assert b"static scratch" in L.moe_last_error()
