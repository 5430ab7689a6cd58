"""GPU parity of the backward pass (ssd_backward) against the fp64 oracle's
reverse-mode gradients (oracle.backward, pinned by finite differences of the
forward).

Every case compares each gradient (dx, ddt, dA, dB, dC, dD, the initial
state's, and with options the dt bias's) by relative L2 at the forward's
tolerances: 1e-4 for float32 inputs, 2e-2 for bf16. Cases cover every state
size with several chunks and a ragged tail, groups, an initial state and a
final-state gradient, the step-size options, the fused forward recompute
and the fused reverse adjoint pass (bf16, Bt*H >= 512), and the 2.7B
layer's shape (one batch row checked).
"""
import numpy as np
import pytest

import oracle
import ssd_workloads as W
from gpu_util import check_units, down, print_case, rel_l2, tol, up

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _ssd():
    import structured_state_space_ssd_amd as ssd
    return ssd


def check_backward(w, with_dfinal=True, batches=None, **option_kw):
    """batches: check only these batch rows of the per-token gradients (the
    oracle then runs on those rows; dA, dD, dbias are compared only when all
    rows are checked)."""
    ssd = _ssd()
    print_case(f"[backward] {w.name} Bt={w.batch} L={w.seqlen} H={w.nheads} G={w.ngroups} "
               f"N={w.dstate} {w.dtype} options={option_kw or 'none'}")
    d = W.generate(w)
    gr = W.generate_grads(w)
    opts = {}
    if option_kw:
        raw = option_kw.pop("raw", False)
        opts = dict(option_kw)
        if raw:
            r = W.generate_dt_raw(w)
            d["dt"] = r["dt"]
            opts["dt_bias"] = r["dt_bias"]
    dfinal = gr["dfinal"] if with_dfinal else None
    gopts = dict(opts)
    if gopts.get("dt_bias") is not None:
        gopts["dt_bias"] = up(gopts["dt_bias"])
    g = ssd.backward(up(d["x"]), up(d["dt"]), up(d["A"]), up(d["B"]), up(d["C"]), up(d["D"]),
                     up(gr["dy"]), init_state=up(d["init"]), dfinal_state=up(dfinal), **gopts)
    torch.cuda.synchronize()
    rows = list(range(w.batch)) if batches is None else list(batches)
    sel = lambda a: None if a is None else np.ascontiguousarray(a[rows])
    ref = oracle.backward(sel(d["x"].val), sel(d["dt"].val), d["A"], sel(d["B"].val),
                          sel(d["C"].val), d["D"], sel(d["init"]), sel(gr["dy"].val), sel(dfinal),
                          **opts)
    errs = {}
    t = tol(w.dtype)
    H, G = w.nheads, w.ngroups
    for k in ("dx", "ddt", "dB", "dC"):
        gk = down(g[k])[rows]
        errs[k] = rel_l2(gk, ref[k])
        # every (batch, head) unit (dB, dC: every (batch, group)) on its own:
        # [Bt, L, U, ...] -> [Bt * U, L, ...]
        nu = G if k in ("dB", "dC") else H
        per = lambda a: np.moveaxis(np.asarray(a).reshape(len(rows), w.seqlen, nu, -1), 2, 1)
        lab = [f"(b {rows[i // nu]}, {'g' if nu == G else 'h'} {i % nu})"
               for i in range(len(rows) * nu)]
        check_units(k, per(gk).reshape(len(rows) * nu, -1), per(ref[k]).reshape(len(rows) * nu, -1),
                    t, lab)
    if d["init"] is not None or with_dfinal:
        gi = down(g["dinit"])[rows]
        errs["dinit"] = rel_l2(gi, ref["dinit"])
        check_units("dinit", gi.reshape(len(rows) * H, -1), np.asarray(ref["dinit"]).reshape(
            len(rows) * H, -1), t)
    if batches is None:
        for k in ("dA", "dD"):
            errs[k] = rel_l2(down(g[k]), ref[k])
        if "dt_bias" in opts:
            errs["ddt_bias"] = rel_l2(down(g["ddt_bias"]), ref["dbias"])
    print_case(f"   errors { {k: f'{v:.2e}' for k, v in errs.items()} }")
    for k, e in errs.items():
        assert e < t, (w.name, k, e)


SWEEP = [("f32", n) for n in (16, 32, 64)] + [("bf16", n) for n in (16, 32, 64, 128, 256)]


@pytest.mark.parametrize("dtype,N", SWEEP, ids=[f"{d}-N{n}" for d, n in SWEEP])
def test_backward_shapes(dtype, N):
    # several of the backward's chunks (64..256 tokens) plus a ragged tail
    w = W.small(f"bwd_{dtype}_N{N}", 2, 600, 4, 64, 2, N, 64, dtype, seed=900 + N, init_std=0.2)
    check_backward(w)


def test_backward_no_init_no_dfinal():
    w = W.small("bwd_plain", 1, 300, 4, 64, 1, 64, 64, "bf16", seed=910)
    check_backward(w, with_dfinal=False)


@pytest.mark.parametrize("L", [1, 37, 128, 129])
def test_backward_short(L):
    check_backward(W.small(f"bwd_short_{L}", 2, L, 2, 64, 1, 32, 64, "f32", seed=920 + L,
                           init_std=0.3))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("opt", ["zoh", "all"])
def test_backward_options(dtype, opt):
    w = W.small(f"bwd_opt_{opt}_{dtype}", 2, 400, 4, 64, 2, 32, 64, dtype, seed=930, init_std=0.2)
    kw = dict(zoh=True) if opt == "zoh" else dict(raw=True, dt_softplus=True,
                                                  dt_limit=(4e-3, 3e-2), zoh=True)
    check_backward(w, **kw)


def test_backward_fused_recompute():
    # Bt*H >= 512: the forward recompute runs stages 2 and 3 as one kernel
    w = W.small("bwd_fused", 8, 300, 64, 64, 4, 64, 64, "bf16", seed=940, init_std=0.2)
    check_backward(w, batches=[0, 5])


def test_backward_fused_adjoint_options_no_dfinal():
    # Bt*H >= 512: the adjoint pass runs as one reverse kernel per (b, h);
    # here with every step-size option and no final-state gradient
    w = W.small("bwd_fused_opt", 8, 333, 64, 64, 2, 64, 64, "bf16", seed=941, init_std=0.2)
    check_backward(w, with_dfinal=False, batches=[1, 6], raw=True, dt_softplus=True,
                   dt_limit=(4e-3, 3e-2), zoh=True)


def test_backward_fused_adjoint_single_chunk():
    w = W.small("bwd_fused_short", 8, 50, 64, 64, 1, 64, 64, "bf16", seed=942, init_std=0.3)
    check_backward(w, batches=[0, 7])


@pytest.mark.parametrize("N", [32, 128, 256])
def test_backward_fused_state_sizes(N):
    # Bt*H >= 512: the recompute and the adjoint pass as one kernel per (b, h)
    # at the other state sizes (phases of 32 tokens at N >= 128, two or three
    # load buffers), several chunks and a ragged end
    w = W.small(f"bwd_fused_N{N}", 8, 301, 64, 64, 4, N, 64, "bf16", seed=945 + N, init_std=0.2)
    check_backward(w, batches=[2, 7])


def test_backward_strong_decay():
    w = W.small("bwd_strong", 1, 500, 4, 64, 1, 32, 64, "f32", seed=950, dt_lo=0.3, dt_hi=2.0)
    check_backward(w)


def test_backward_mamba2_2p7b_full():
    """The 2.7B layer's shape, every batch row and head (dx, ddt, dB, dC,
    dinit, dA, dD)."""
    w = W.WORKLOADS["mamba2_2.7b"]
    check_backward(w, with_dfinal=True)


def test_backward_errors():
    ssd = _ssd()
    x = torch.zeros((1, 10, 2, 64), dtype=torch.float32, device="cuda")
    dt = torch.zeros((1, 10, 2), dtype=torch.float32, device="cuda")
    A = torch.zeros(2, dtype=torch.float32, device="cuda")
    B = torch.zeros((1, 10, 1, 128), dtype=torch.float32, device="cuda")  # fp32 N 128
    with pytest.raises(ssd.SSDError):
        ssd.backward(x, dt, A, B, B.clone(), None, x.clone())
    with pytest.raises(ValueError):
        ssd.backward(x, dt, A, B[..., :64].contiguous(), B[..., :64].contiguous(), None,
                     x[:, :5].contiguous())


@pytest.mark.parametrize("dtype,N", [("bf16", 48), ("f32", 48), ("bf16", 96), ("bf16", 192)])
def test_backward_padded_dstate(dtype, N):
    # state sizes outside the kernels' set: B, C, the states zero-padded to the
    # next kernel size, dB, dC and the initial state's gradient cut back
    w = W.small(f"bwd_pad_{dtype}_N{N}", 2, 333, 4, 64, 2, N, 64, dtype, seed=1400 + N,
                init_std=0.2)
    check_backward(w)
