"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every case runs the same seeded inputs through the library and the oracle and
compares relative L2 at the stated tolerances (1e-4 float32, 2e-2 bf16, 1e-3
for the decode state). Each forward case is also run with D = 0, because the
D x term dominates y and would otherwise hide errors in the SSM part.
"""
import math

import numpy as np
import pytest

import oracle
import ssd_workloads as W
from gpu_util import check_units, down, print_case, rel_l2, tol, units_view, up

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _ssd():
    import structured_state_space_ssd_amd as ssd
    return ssd


def run_forward(w, d, D, init, opts=None):
    ssd = _ssd()
    opts = dict(opts or {})
    if opts.get("dt_bias") is not None:
        opts["dt_bias"] = up(opts["dt_bias"])
    y, fs = ssd.forward(up(d["x"]), up(d["dt"]), up(d["A"]), up(d["B"]), up(d["C"]),
                        None if D is None else up(D), chunk=w.chunk, init_state=up(init),
                        return_final_state=True, **opts)
    torch.cuda.synchronize()
    return y, fs


def plan(w):
    """Segments of the single-pass forward for this workload (0: stage kernels)."""
    return _ssd().forward_plan(w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate,
                               w.chunk, torch.bfloat16 if w.dtype == "bf16" else torch.float32)


def with_options(w, d, raw=False, dt_softplus=False, dt_limit=None, zoh=False):
    """The option set for a case: raw=True swaps in pre-softplus dt values and
    a per-head bias (ssd_workloads.generate_dt_raw); returns the keyword
    arguments shared by the oracle and the library."""
    opts = dict(dt_softplus=dt_softplus, dt_limit=dt_limit, zoh=zoh, dt_bias=None)
    if raw:
        r = W.generate_dt_raw(w)
        d["dt"] = r["dt"]
        opts["dt_bias"] = r["dt_bias"]
    return opts


def check_forward(w, units=None, init=None, both_D=True, **option_kw):
    """Compare y and the final state with the oracle (all units or a sample).
    ``option_kw`` (see with_options) turns on step-size preprocessing and the
    zero-order-hold input weight on both sides."""
    print_case(f"[forward] {w.name} Bt={w.batch} L={w.seqlen} H={w.nheads} G={w.ngroups} "
               f"N={w.dstate} Q={w.chunk} {w.dtype} units={'all' if units is None else len(units)} "
               f"options={option_kw or 'none'}")
    d = W.generate(w)
    opts = with_options(w, d, **option_kw) if option_kw else None
    if init is None:
        init = d["init"]
    H = w.nheads
    uu = np.arange(w.batch * H) if units is None else np.asarray(units)
    # oracle without D; the D x term is added exactly in float64 (y is linear in it)
    y0, s0, _ = oracle.forward(d["x"].val, d["dt"].val, d["A"], d["B"].val, d["C"].val, None,
                               init, units=None if units is None else uu, **(opts or {}))
    xv = units_view(d["x"].val, uu, H).astype(np.float64)
    Dv = d["D"].astype(np.float64)[uu % H][:, None, None]
    errs = {}
    t = tol(w.dtype)
    labels = [f"(b {u // H}, h {u % H})" for u in uu]
    for with_D in ([True, False] if both_D else [True]):
        y, fs = run_forward(w, d, d["D"] if with_D else None, init, opts)
        yg = units_view(down(y), uu, H)
        yref = y0 + Dv * xv if with_D else y0
        tag = f"y{'_D' if with_D else '_noD'}"
        errs[tag] = rel_l2(yg, yref)
        # every (batch, head) unit on its own, too
        errs[tag + "_worst_unit"] = check_units(tag, yg, yref, t, labels, part=y0)
        fsg = down(fs).reshape(-1, w.headdim, w.dstate)[uu]
        errs["state"] = rel_l2(fsg, s0)
        errs["state_worst_unit"] = check_units("state", fsg, s0, t, labels)
        del y, fs, yg
    print_case(f"   errors {errs}")
    for k, e in errs.items():
        assert e < t, (w.name, k, e)
    return errs


# ---------------------------------------------------------------- named workloads

def test_tiny_f32():
    check_forward(W.WORKLOADS["tiny_f32"])


def test_mamba2_2p7b_full():
    check_forward(W.WORKLOADS["mamba2_2.7b"])


def test_large_state_full():
    check_forward(W.WORKLOADS["large_state"])


def test_long_seq_full():
    # every one of the 80 heads (8 groups), y with and without D, the final state
    check_forward(W.WORKLOADS["long_seq"])


def test_decode_64_steps():
    # every one of the 256 x 80 (batch, head) units
    _decode(W.WORKLOADS["decode"], zero_init=False, nunits=None)


def test_decode_64_steps_zero_init():
    _decode(W.WORKLOADS["decode"], zero_init=True, nunits=None)


def _decode(w, zero_init, nunits=512, **option_kw):
    ssd = _ssd()
    print_case(f"[decode] {w.name} Bt={w.batch} H={w.nheads} N={w.dstate} steps={w.seqlen} "
               f"zero_init={zero_init} options={option_kw or 'none'}")
    d = W.generate(w)
    opts = with_options(w, d, **option_kw) if option_kw else {}
    gopts = dict(opts)
    if gopts.get("dt_bias") is not None:
        gopts["dt_bias"] = up(gopts["dt_bias"])
    H, P, N = w.nheads, w.headdim, w.dstate
    rng = np.random.default_rng(123)
    units = (np.arange(w.batch * H) if nunits is None else
             np.sort(rng.choice(w.batch * H, size=nunits, replace=False)))
    init = np.zeros_like(d["init"]) if zero_init else d["init"]
    state = up(init)
    st_o = np.ascontiguousarray(init.reshape(-1, P, N)[units].astype(np.float64))
    X, DT, Bv, Cv = up(d["x"]), up(d["dt"]), up(d["B"]), up(d["C"])
    A, D = up(d["A"]), up(d["D"])
    ys, yos = [], []
    for t in range(w.seqlen):
        y = ssd.step(state, X[t], DT[t], A, Bv[t], Cv[t], D, **gopts)
        ys.append(down(y).reshape(-1, P)[units])
        yos.append(oracle.step(st_o, d["x"].val[t], d["dt"].val[t], d["A"], d["B"].val[t],
                               d["C"].val[t], d["D"], units=units, **opts))
    torch.cuda.synchronize()
    yg, yr = np.stack(ys, axis=1), np.stack(yos, axis=1)  # [U, steps, P]
    ey = rel_l2(yg, yr)
    sg = down(state).reshape(-1, P, N)[units]
    es = rel_l2(sg, st_o)
    print_case(f"   rel_l2 y={ey:.3e} state={es:.3e}")
    labels = [f"(b {u // w.nheads}, h {u % w.nheads})" for u in units]
    check_units("y", yg, yr, tol(w.dtype), labels)
    check_units("state", sg, st_o, 1e-3, labels)
    assert ey < tol(w.dtype) and es < 1e-3


# ---------------------------------------------------------------- sweeps and edge cases

SWEEP = [(n, q, dt) for dt in ("f32", "bf16") for n in (16, 32, 64, 128, 256) for q in (64, 128, 256)]


@pytest.mark.parametrize("N,Q,dtype", SWEEP, ids=[f"N{n}-Q{q}-{d}" for n, q, d in SWEEP])
def test_sweep_shapes(N, Q, dtype):
    # several chunks plus a ragged tail; 2 groups; non-zero initial state
    w = W.small(f"sweep_N{N}_Q{Q}_{dtype}", 2, 2 * Q + 37, 4, 64, 2, N, Q, dtype,
                seed=100 + N + Q, init_std=0.2)
    check_forward(w)


@pytest.mark.parametrize("L,Q", [(1, 64), (50, 64), (64, 64), (65, 64), (127, 128), (300, 256)])
def test_short_and_ragged(L, Q):
    check_forward(W.small(f"ragged_L{L}_Q{Q}", 3, L, 2, 64, 1, 64, Q, "bf16", seed=200 + L))


def test_groups_8():
    check_forward(W.small("groups8", 1, 600, 16, 64, 8, 128, 256, "bf16", seed=301, init_std=0.1))


def test_strong_decay_and_large_dt():
    # dt up to 2 with A down to -16: within-chunk log-decay far below fp32 exp range
    check_forward(W.small("strong", 2, 512, 4, 64, 1, 64, 256, "f32", seed=302, dt_lo=0.5, dt_hi=2.0))


def test_slow_decay_long():
    check_forward(W.small("slow", 1, 4096, 4, 64, 1, 64, 128, "f32", seed=303, dt_lo=1e-5, dt_hi=1e-4))


# ------------------------------------------------- fused stages 2 + 3 (bf16, Bt*H >= 512)
#
# With enough (batch, head) units the bf16 forward runs the chunk states and
# the state passing as one kernel per (batch, head); these cases reach it at
# sizes the oracle finishes quickly, with ragged ends, an initial state,
# several groups and every state size and chunk length. (With N = 64 and a
# multiple of 8 heads the whole forward runs as the single-pass kernel
# instead: see the next section.)

@pytest.mark.parametrize("N,Q", [(16, 64), (32, 128), (64, 256), (128, 128), (256, 64), (64, 64),
                                 (128, 256)])
def test_fused_state_path(N, Q):
    # 68 heads (not a multiple of 8): the stage kernels run at every N
    w = W.small(f"fused_N{N}_Q{Q}", 8, 2 * Q + 45, 68, 64, 4, N, Q, "bf16",
                seed=600 + N + Q, init_std=0.2)
    assert w.batch * w.nheads >= 512 and plan(w) == 0
    check_forward(w)


def test_fused_state_path_single_chunk_short():
    # one partial chunk only: the state passing reduces to H_1 = exp(s_end) H_0 + S_0
    check_forward(W.small("fused_short", 16, 37, 32, 64, 1, 64, 256, "bf16", seed=620, init_std=0.3))


# --------------------- single-pass forward (bf16, N 64 or 128, heads a multiple of 8)
#
# One workgroup per (batch, head) walks the sequence in 64-token blocks with
# the state in registers (these cases have enough (batch, head) pairs for one
# segment; the segmented form follows further down). Cases: a single token, one partial block, exactly
# one block, one block plus one token, several blocks with a ragged end (the
# last block ending inside an even 16-token row tile, and inside an odd one:
# 84 and 247, where an odd tile's diagonal slice takes its unmasked path); an
# initial state; several groups; every chunk argument (it does not change the
# kernel's blocks, only the rounding order against the oracle).

@pytest.mark.parametrize("L", [1, 37, 64, 65, 84, 200, 247, 1000])
def test_onepass_lengths(L):
    w = W.small(f"onepass_L{L}", 8, L, 64, 64, 4, 64, 256, "bf16", seed=800 + L, init_std=0.2)
    assert w.batch * w.nheads >= 512
    check_forward(w)


@pytest.mark.parametrize("Q", [64, 128])
def test_onepass_chunk_argument(Q):
    w = W.small(f"onepass_Q{Q}", 4, 3 * Q + 11, 128, 64, 1, 64, Q, "bf16", seed=810 + Q)
    check_forward(w)


def test_onepass_groups_no_init():
    check_forward(W.small("onepass_g8", 2, 333, 256, 64, 8, 64, 256, "bf16", seed=820))


@pytest.mark.parametrize("name", ["all_zoh", "softplus_bias", "softplus_bias_clamp", "zoh"])
def test_onepass_options(name):
    w = W.small(f"onepass_opt_{name}", 8, 2 * 64 + 29, 64, 64, 2, 64, 256, "bf16", seed=830,
                init_std=0.2)
    check_forward(w, **OPTION_SETS[name])


def test_onepass_one_head_per_group():
    # ngroups = nheads: every workgroup reads its own B and C rows
    check_forward(W.small("onepass_g64", 8, 150, 64, 64, 64, 64, 128, "bf16", seed=860,
                          init_std=0.2))


def test_onepass_strong_decay():
    # steps up to 2 with A down to -16: within a 64-token block the log-decay
    # spans far more than fp32's exponent range (every decay factor the
    # kernel forms must stay <= 1, with no inf times 0)
    w = W.small("onepass_strong", 8, 300, 64, 64, 2, 64, 256, "bf16", seed=850,
                dt_lo=0.5, dt_hi=2.0, init_std=0.2)
    check_forward(w)


def test_onepass_long_sequence_sampled():
    # 16384 tokens (256 blocks per (batch, head)), x about 1 GB; the oracle
    # checks a first, a middle and a last unit, across batch rows and groups
    w = W.small("onepass_long", 8, 16384, 64, 64, 4, 64, 256, "bf16", seed=880, init_std=0.1,
                dt_lo=1e-4, dt_hi=1e-2)
    check_forward(w, units=[0, 64 * 3 + 37, 8 * 64 - 1], both_D=False)


def test_onepass_misaligned_dt_falls_back():
    # dt 2 bytes off a 16-byte boundary: the single-pass kernel reads dt as
    # 16-byte pieces, so the forward takes the stage kernels instead
    ssd = _ssd()
    w = W.small("onepass_dt_off", 8, 130, 64, 64, 2, 64, 128, "bf16", seed=870)
    d = W.generate(w)
    dtg = up(d["dt"])
    buf = torch.empty(dtg.numel() + 8, dtype=dtg.dtype, device=dtg.device)
    dt_off = buf[1:1 + dtg.numel()].view(dtg.shape)
    dt_off.copy_(dtg)
    assert dt_off.data_ptr() % 16 != 0
    y = ssd.forward(up(d["x"]), dt_off, up(d["A"]), up(d["B"]), up(d["C"]), up(d["D"]),
                    chunk=w.chunk)
    torch.cuda.synchronize()
    y0, _, _ = oracle.forward(d["x"].val, d["dt"].val, d["A"], d["B"].val, d["C"].val, d["D"],
                              None)
    e = rel_l2(units_view(down(y), np.arange(w.batch * w.nheads), w.nheads), y0)
    print_case(f"[forward] misaligned dt: rel_l2(y) = {e:.3e}")
    assert e < tol(w.dtype), e


# ----------------------- single-pass forward over segments (few (batch, head) pairs)
#
# With fewer (batch, head) pairs than fill the GPU, each sequence is cut into
# S segments of whole 64-token blocks: a first kernel computes each segment's
# state from zero, the single-pass kernel starts each segment from the state
# the earlier segments pass on. Cases: N 64 and 128; S from 2 to 8, ragged
# last segments, an initial state and none, several groups (every step-size
# option further down); a single segment at N 128 (enough pairs) and sequences too short to
# cut.

@pytest.mark.parametrize("N", [64, 128, 256])
@pytest.mark.parametrize("L", [37 * 64 + 13, 8 * 64, 1000])
def test_segments(N, L):
    w = W.small(f"seg_N{N}_L{L}", 1, L, 16, 64, 2, N, 256, "bf16", seed=900 + L + N,
                init_std=0.2)
    S = plan(w)
    print_case(f"   segments {S}")
    assert S > 1
    check_forward(w)


def test_segments_many_groups_no_init():
    w = W.small("seg_g8", 2, 3000, 8, 64, 8, 128, 128, "bf16", seed=930)
    assert plan(w) > 1
    check_forward(w)


def test_segments_strong_decay():
    # fast decay: each segment's contribution to the next almost vanishes
    w = W.small("seg_strong", 1, 2000, 16, 64, 1, 64, 256, "bf16", seed=950, init_std=0.2,
                dt_lo=0.2, dt_hi=1.0)
    assert plan(w) > 1
    check_forward(w, both_D=False)


@pytest.mark.parametrize("N", [64, 128])
@pytest.mark.parametrize("G", [8, 3])
def test_segments_heads_per_group(N, G):
    # the segment-state kernel takes two heads of a group per workgroup where a
    # group has an even number of heads (G 3: eight per group), one otherwise
    # (G 8: three per group)
    w = W.small(f"seg_hpg_N{N}_G{G}", 1, 1500, 24, 64, G, N, 256, "bf16", seed=940 + N + G,
                init_std=0.2)
    assert plan(w) > 1
    check_forward(w)


@pytest.mark.parametrize("L", [1, 100, 255])
def test_segments_too_short_to_cut(L):
    w = W.small(f"seg_short_L{L}", 1, L, 8, 64, 1, 128, 64, "bf16", seed=960 + L, init_std=0.2)
    assert plan(w) == 1
    check_forward(w)


def test_onepass_n128_one_segment():
    w = W.small("onepass_n128", 8, 333, 64, 64, 4, 128, 256, "bf16", seed=970, init_std=0.2)
    assert plan(w) == 1
    check_forward(w)


def test_onepass_n256_one_segment():
    w = W.small("onepass_n256", 8, 333, 32, 64, 4, 256, 128, "bf16", seed=971, init_std=0.2)
    assert plan(w) == 1
    check_forward(w)


def test_onepass_n256_options_segments():
    w = W.small("onepass_n256_opt", 2, 1100, 8, 64, 2, 256, 64, "bf16", seed=972, init_std=0.2)
    assert plan(w) > 1
    check_forward(w, both_D=False, raw=True, dt_softplus=True, dt_limit=(4e-3, 3e-2), zoh=True)


def test_heads_not_multiple_of_8_many_units():
    # 9 x 60 units but 60 heads: the separate-stage path (its fused state kernel)
    check_forward(W.small("h60", 9, 300, 60, 64, 3, 64, 128, "bf16", seed=840, init_std=0.2))


# ------------------------------------ step-size preprocessing and zero-order hold
#
# dt_bias + softplus + clamp (the selection mechanism's step size) and the
# zero-order-hold input weight (exp(dt A) - 1) / A, alone and together, on the
# separate-stage path (f32, and bf16 with few units), the fused bf16 path and
# the decode step. The clamp bounds are hit on both sides.

OPTION_SETS = {
    "zoh": dict(zoh=True),
    "softplus_bias": dict(raw=True, dt_softplus=True),
    "softplus_bias_clamp": dict(raw=True, dt_softplus=True, dt_limit=(4e-3, 3e-2)),
    "all_zoh": dict(raw=True, dt_softplus=True, dt_limit=(4e-3, 3e-2), zoh=True),
}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", sorted(OPTION_SETS))
def test_options_forward(name, dtype):
    w = W.small(f"opt_{name}_{dtype}", 2, 2 * 128 + 37, 4, 64, 2, 64, 128, dtype,
                seed=700 + len(name), init_std=0.2)
    check_forward(w, **OPTION_SETS[name])


@pytest.mark.parametrize("name", ["zoh", "all_zoh"])
def test_options_fused_state_path(name):
    w = W.small(f"opt_fused_{name}", 8, 2 * 256 + 45, 68, 64, 4, 64, 256, "bf16", seed=710,
                init_std=0.2)
    assert w.batch * w.nheads >= 512 and plan(w) == 0
    check_forward(w, **OPTION_SETS[name])


@pytest.mark.parametrize("name", sorted(OPTION_SETS))
def test_segments_options(name):
    # the single-pass forward over segments (N 128), every option set
    w = W.small(f"seg_opt_{name}", 2, 1500, 8, 64, 2, 128, 256, "bf16", seed=940,
                init_std=0.2)
    assert plan(w) > 1
    check_forward(w, both_D=False, **OPTION_SETS[name])


def test_options_strong_decay_zoh():
    # large steps: the zoh weight (1 - e^{dt A}) / |A| saturates at 1/|A|, far from dt
    check_forward(W.small("opt_strong_zoh", 2, 300, 4, 64, 1, 64, 128, "f32", seed=711,
                          dt_lo=0.5, dt_hi=2.0), zoh=True)


def test_mamba2_2p7b_all_options():
    # every (batch, head) unit of the 2.7B shape with every option on
    check_forward(W.WORKLOADS["mamba2_2.7b"], both_D=False, **OPTION_SETS["all_zoh"])


@pytest.mark.parametrize("name", ["zoh", "all_zoh"])
def test_options_decode(name):
    _decode(W.WORKLOADS["decode"], zero_init=False, nunits=256, **OPTION_SETS[name])


def test_options_decode_f32():
    w = W.Workload("decode_f32_opts", 16, 12, 8, 64, 2, 64, 0, "f32", 1 / 8, 1e-3, 1e-1,
                   init_std=0.2, decode=True, seed=712)
    _decode(w, zero_init=False, nunits=64, **OPTION_SETS["all_zoh"])


def test_segments_many_n256_sampled():
    # batch 1, 16 heads, 16384 tokens at N 256: many segments and pieces of the
    # eight-wavefront kernels, an initial state; sampled heads against the oracle
    w = W.small("seg_many_n256", 1, 16384, 16, 64, 2, 256, 128, "bf16", seed=980, init_std=0.1,
                dt_lo=1e-4, dt_hi=1e-2)
    S = plan(w)
    print_case(f"   segments {S}")
    assert S >= 8
    check_forward(w, units=[0, 7, 8, 15], both_D=False)


# ------------------------------------------------- workspace bounds of the segmented path
#
# The segment-state kernel writes one float32 state and decay per piece of
# every (batch, head); the plan sizes the workspace to exactly that. Canary
# bytes after an exact-size workspace must come back untouched (they did not
# before the piece count was taken per (batch, head) times their number).

@pytest.mark.parametrize("L,H,G,N", [(2000, 16, 1, 64), (1000, 16, 2, 64), (1000, 16, 2, 128),
                                     (37 * 64 + 13, 16, 2, 256), (700, 8, 2, 128)])
def test_segments_workspace_canary(L, H, G, N):
    ssd = _ssd()
    w = W.small(f"canary_L{L}_N{N}", 1, L, H, 64, G, N, 256, "bf16", seed=990 + N, init_std=0.2)
    d = W.generate(w)
    g = {k: up(d[k]) for k in ("x", "dt", "A", "B", "C", "D", "init")}
    p = ssd.plan_info(w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate, w.chunk,
                      torch.bfloat16, g["dt"])
    print_case(f"   plan {p}")
    assert p["segments"] > 1 and p["workspace_bytes"] > 0
    need, pad = p["workspace_bytes"], 1 << 20
    ws = torch.full((need + pad,), 0xA5, dtype=torch.uint8, device="cuda")
    y, fs = ssd.forward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], chunk=w.chunk,
                        init_state=g["init"], return_final_state=True, workspace=ws)
    torch.cuda.synchronize()
    assert bool((ws[need:] == 0xA5).all()), "the forward wrote past its workspace"
    y0, s0, _ = oracle.forward(d["x"].val, d["dt"].val, d["A"], d["B"].val, d["C"].val, d["D"],
                               d["init"])
    e = rel_l2(units_view(down(y), np.arange(H), H), y0)
    print_case(f"   rel_l2(y) = {e:.3e}")
    assert e < tol(w.dtype)


def test_varlen_workspace_canary():
    ssd = _ssd()
    w = W.small("canary_varlen", 1, 3000, 16, 64, 2, 128, 256, "bf16", seed=995)
    cu = W.packed_cu_seqlens(w.seqlen, 700, seed=996)
    d = W.generate(w)
    g = {k: up(d[k]) for k in ("x", "dt", "A", "B", "C", "D")}
    need = int(ssd._native.lib.ssd_forward_varlen_workspace_size(
        w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate, w.chunk, 1))
    ws = torch.full((need + (1 << 20),), 0x5A, dtype=torch.uint8, device="cuda")
    y, ss = ssd.forward_varlen(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"],
                               torch.from_numpy(cu).cuda(), chunk=w.chunk, return_seq_states=True,
                               workspace=ws)
    torch.cuda.synchronize()
    assert bool((ws[need:] == 0x5A).all()), "the packed forward wrote past its workspace"
    y0, st0 = oracle.forward_varlen(d["x"].val, d["dt"].val, d["A"], d["B"].val, d["C"].val,
                                    d["D"], cu)
    e = rel_l2(down(y)[0].transpose(1, 0, 2), y0)
    print_case(f"   rel_l2(y) = {e:.3e}")
    assert e < tol(w.dtype)


# ------------------------------------- state sizes outside the kernels' own set
#
# Any multiple of 16 up to 256 runs the kernels of the next of 16, 32, 64,
# 128, 256 on zero-padded copies of B, C and the states (the padded columns
# add exact zeros). Cases reach the single-pass kernel (bf16, heads a multiple
# of 8, with and without segments) and the stage kernels (float32, and bf16
# with 4 heads), with an initial state and the final state compared.

PADDED = [(48, "bf16", 8, 64), (48, "f32", 1, 4), (80, "bf16", 1, 16), (96, "bf16", 4, 4),
          (112, "f32", 2, 4), (144, "bf16", 1, 8), (192, "bf16", 2, 32), (240, "bf16", 1, 4)]


@pytest.mark.parametrize("N,dtype,Bt,H", PADDED, ids=[f"N{n}-{d}-B{b}-H{h}" for n, d, b, h in PADDED])
def test_padded_dstate_forward(N, dtype, Bt, H):
    w = W.small(f"pad_N{N}_{dtype}_B{Bt}_H{H}", Bt, 2 * 128 + 77, H, 64, 2, N, 128, dtype,
                seed=1300 + N + Bt, init_std=0.2)
    p = _ssd().plan_info(w.batch, w.seqlen, w.nheads, 64, w.ngroups, N, w.chunk,
                         torch.bfloat16 if dtype == "bf16" else torch.float32)
    print_case(f"   plan {p}")
    assert p["kernel_dstate"] > N
    check_forward(w)


def test_padded_dstate_segments_with_options():
    w = W.small("pad_seg_opts", 1, 3000, 8, 64, 2, 96, 256, "bf16", seed=1350, init_std=0.2)
    assert plan(w) > 1
    check_forward(w, both_D=False, **OPTION_SETS["all_zoh"])


@pytest.mark.parametrize("N", [48, 96, 240])
def test_padded_dstate_decode(N):
    w = W.Workload(f"decode_N{N}", 8, 16, 8, 64, 2, N, 0, "bf16", 1 / math.sqrt(N), 1e-3, 1e-1,
                   init_std=0.1, decode=True, seed=1360 + N)
    _decode(w, zero_init=False, nunits=None)
