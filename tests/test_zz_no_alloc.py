"""ssd_forward_static (the allocation-free forward: its scratch is a fixed
device array inside the library) through the C ABI, against ssd_forward_ex
with a caller workspace on the same inputs, and against the fp64 oracle.

Two calls in a row, the second with a smaller input (the array keeps the
first call's contents), then a float32 forward on the stage kernels, whose
whole workspace lives in the array. Both entry points run the same kernels
with the same plan, so their outputs must agree bit for bit."""
import ctypes

import numpy as np
import pytest

import oracle
import ssd_workloads as W
from gpu_util import down, print_case, rel_l2, tol, units_view, up

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

STATIC_BYTES = 32 << 20


def _lib():
    from structured_state_space_ssd_amd import _native
    return _native


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _run(w, d, static):
    nat = _lib()
    g = {k: up(d[k]) for k in ("x", "dt", "A", "B", "C", "D", "init")}
    dtc = 1 if w.dtype == "bf16" else 0
    y = torch.full_like(g["x"], float("nan"))
    fs = torch.full((w.batch, w.nheads, w.headdim, w.dstate), float("nan"), dtype=torch.float32,
                    device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [_p(g["x"]), _p(g["dt"]), _p(g["A"]), _p(g["B"]), _p(g["C"]), _p(g["D"]), w.batch,
            w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate, w.chunk, dtc, _p(g["init"]),
            _p(y), _p(fs)]
    if static:
        rc = nat.lib.ssd_forward_static(*args, None, stream)
    else:
        p = nat.SsdPlan()
        assert nat.lib.ssd_forward_plan_info(w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups,
                                             w.dstate, w.chunk, dtc, _p(g["dt"]),
                                             ctypes.byref(p)) == 0
        ws = torch.empty(max(1, p.workspace_bytes), dtype=torch.uint8, device="cuda")
        rc = nat.lib.ssd_forward_ex(*args, _p(ws), ws.numel(), None, stream, None)
    assert rc == 0, nat.lib.ssd_strerror(rc)
    torch.cuda.synchronize()
    return y, fs


CASES = [
    # (name, batch, L, H, G, N, Q, dtype): segmented single-pass at N 128, then a
    # smaller segmented one at N 64, then float32 on the stage kernels
    ("static_seg_n128", 1, 3000, 16, 2, 128, 256, "bf16"),
    ("static_seg_n64_smaller", 1, 1000, 8, 1, 64, 128, "bf16"),
    ("static_stages_f32", 2, 300, 4, 2, 64, 64, "f32"),
]


def test_forward_static_matches_forward_ex():
    import structured_state_space_ssd_amd as ssd
    for k, (name, Bt, L, H, G, N, Q, dt) in enumerate(CASES):
        w = W.small(name, Bt, L, H, 64, G, N, Q, dt, seed=1200 + k, init_std=0.2)
        p = ssd.plan_info(Bt, L, H, 64, G, N, Q, torch.bfloat16 if dt == "bf16" else torch.float32)
        print_case(f"[static] {name}: plan {p}")
        assert 0 < p["workspace_bytes"] <= STATIC_BYTES
        d = W.generate(w)
        ys, fss = _run(w, d, static=True)
        ye, fse = _run(w, d, static=False)
        assert torch.equal(ys, ye) and torch.equal(fss, fse), name
        y0, s0, _ = oracle.forward(d["x"].val, d["dt"].val, d["A"], d["B"].val, d["C"].val,
                                   d["D"], d["init"])
        ey = rel_l2(units_view(down(ys), np.arange(Bt * H), H), y0)
        es = rel_l2(down(fss).reshape(-1, 64, N), s0)
        print_case(f"   bitwise equal to ssd_forward_ex; rel_l2 y={ey:.3e} state={es:.3e}")
        assert ey < tol(dt) and es < tol(dt)
