"""GPU parity of packed variable-length sequences (ssd_forward_varlen) against
the fp64 oracle (oracle.forward_varlen: the recurrence with the state reset
where each sequence begins).

Every case compares y (with D and with D = 0) and every sequence's final
state at the forward's tolerances. Boundaries are placed on chunk starts, on
chunk ends, inside chunks and inside 32-token slices, with empty and
one-token sequences; the mixes of lengths come from
ssd_workloads.packed_cu_seqlens.
"""
import numpy as np
import pytest

import oracle
import ssd_workloads as W
from gpu_util import check_units, down, print_case, rel_l2, tol, unit_rel_l2, up

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _ssd():
    import structured_state_space_ssd_amd as ssd
    return ssd


def check_varlen(w, cu, units=None, **option_kw):
    """w: a batch-1 workload (x [1,L,H,P] ...); cu: int32 offsets."""
    ssd = _ssd()
    cu = np.asarray(cu, np.int32)
    print_case(f"[varlen] {w.name} L={w.seqlen} H={w.nheads} G={w.ngroups} N={w.dstate} "
               f"Q={w.chunk} {w.dtype} nseq={cu.size - 1} options={option_kw or 'none'}")
    assert w.batch == 1 and cu[0] == 0 and cu[-1] == w.seqlen
    d = W.generate(w)
    opts = {}
    if option_kw:
        raw = option_kw.pop("raw", False)
        opts = dict(option_kw)
        if raw:
            r = W.generate_dt_raw(w)
            d["dt"] = r["dt"]
            opts["dt_bias"] = r["dt_bias"]
    H, P, N = w.nheads, w.headdim, w.dstate
    uu = np.arange(H) if units is None else np.asarray(units)
    y0, st0 = oracle.forward_varlen(d["x"].val, d["dt"].val, d["A"], d["B"].val, d["C"].val, None,
                                    cu, units=None if units is None else uu, **opts)
    gopts = dict(opts)
    if gopts.get("dt_bias") is not None:
        gopts["dt_bias"] = up(gopts["dt_bias"])
    cu_g = torch.from_numpy(cu).cuda()
    errs = {}
    for with_D in (True, False):
        y, ss = ssd.forward_varlen(up(d["x"]), up(d["dt"]), up(d["A"]), up(d["B"]), up(d["C"]),
                                   up(d["D"]) if with_D else None, cu_g, chunk=w.chunk,
                                   return_seq_states=True, **gopts)
        torch.cuda.synchronize()
        yg = down(y)[0].transpose(1, 0, 2)[uu]  # [U, L, P]
        yref = y0 + (d["D"].astype(np.float64)[uu][:, None, None] *
                     d["x"].val[0].transpose(1, 0, 2)[uu]) if with_D else y0
        tag = "y_D" if with_D else "y_noD"
        errs[tag] = rel_l2(yg, yref)
        # every (sequence, head) unit on its own: [U, L, P] -> one row per pair
        # (y = the state-space part y0 + D x: measured against the larger of
        # the two, see gpu_util.unit_rel_l2)
        pg, pr, p0, lab = [], [], [], []
        for k in range(cu.size - 1):
            if cu[k + 1] > cu[k]:
                pg += list(yg[:, cu[k]:cu[k + 1]])
                pr += list(yref[:, cu[k]:cu[k + 1]])
                p0 += list(y0[:, cu[k]:cu[k + 1]])
                lab += [f"(seq {k}, h {u})" for u in uu]
        e = [float(unit_rel_l2(a[None], b[None], c[None])[0]) for a, b, c in zip(pg, pr, p0)]
        worst = int(np.argmax(e))
        print_case(f"   per-unit {tag}: worst {e[worst]:.3e} at {lab[worst]} of {len(e)}")
        assert e[worst] < tol(w.dtype), (tag, lab[worst], e[worst])
        sg = down(ss).transpose(1, 0, 2, 3)[uu]  # [U, nseq, P, N]
        errs["states"] = rel_l2(sg, st0)
        nonempty = np.flatnonzero(np.diff(cu) > 0)
        check_units("states", sg[:, nonempty].reshape(-1, w.headdim * w.dstate),
                    np.asarray(st0)[:, nonempty].reshape(-1, w.headdim * w.dstate), tol(w.dtype),
                    [f"(h {u}, seq {k})" for u in uu for k in nonempty])
        # empty sequences have exactly zero states
        empty = np.flatnonzero(np.diff(cu) == 0)
        assert np.all(sg[:, empty] == 0)
    print_case(f"   errors {errs}")
    for k, e in errs.items():
        assert e < tol(w.dtype), (w.name, k, e)


def _w(name, L, H, G, N, Q, dtype, seed):
    return W.small(name, 1, L, H, 64, G, N, Q, dtype, seed=seed)


# boundaries at chunk starts (64, 256), at a chunk end (127|128), inside
# chunks and slices, an empty sequence, one-token sequences, a long tail
EXPLICIT = [0, 1, 1, 9, 64, 65, 128, 200, 256, 300, 513, 700]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_varlen_explicit_boundaries(dtype):
    check_varlen(_w(f"vl_explicit_{dtype}", 700, 4, 2, 64, 64, dtype, 801), EXPLICIT)


MIX = [(n, q, dt) for dt in ("f32", "bf16") for n in (16, 64, 128, 256) for q in (64, 256)]


@pytest.mark.parametrize("N,Q,dtype", MIX, ids=[f"N{n}-Q{q}-{d}" for n, q, d in MIX])
def test_varlen_length_mix(N, Q, dtype):
    # lengths from 1 to 300 over several chunks: the bf16 scan's pair kernel
    # (N <= 64) and one-per-compute-unit kernel (N >= 128) and the float kernel
    L = 3 * Q + 77
    cu = W.packed_cu_seqlens(L, 300, seed=810 + N + Q)
    check_varlen(_w(f"vl_mix_N{N}_Q{Q}_{dtype}", L, 4, 2, N, Q, dtype, 820 + N + Q), cu)


def test_varlen_many_short_sequences():
    # every sequence shorter than a 32-token slice: masks in every slice
    L = 512
    cu = W.packed_cu_seqlens(L, 12, seed=830)
    assert cu.size > 60
    check_varlen(_w("vl_short_bf16", L, 4, 1, 64, 256, "bf16", 831), cu)
    check_varlen(_w("vl_short_f32", L, 4, 1, 64, 128, "f32", 832), cu)


def test_varlen_single_sequence_equals_forward():
    """One sequence is the plain forward on the stage kernels (6 heads: not the
    single-pass kernel): the masked kernels compute the same values in the
    same order, so the outputs are bitwise equal."""
    ssd = _ssd()
    for dtype, N, Q in (("bf16", 64, 256), ("bf16", 128, 256), ("f32", 64, 128)):
        w = _w(f"vl_single_{dtype}_{N}", 777, 6, 2, N, Q, dtype, 840 + N)
        assert ssd.forward_plan(w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate,
                                Q, torch.bfloat16 if dtype == "bf16" else torch.float32) == 0
        d = W.generate(w)
        g = {k: up(d[k]) for k in ("x", "dt", "A", "B", "C", "D")}
        cu = torch.tensor([0, w.seqlen], dtype=torch.int32, device="cuda")
        y1, s1 = ssd.forward_varlen(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], cu,
                                    chunk=Q, return_seq_states=True)
        y2, s2 = ssd.forward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], chunk=Q,
                             return_final_state=True)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2), dtype
        assert rel_l2(down(s1[0]), down(s2[0])) < tol(dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_varlen_with_options(dtype):
    L = 600
    cu = W.packed_cu_seqlens(L, 200, seed=850)
    check_varlen(_w(f"vl_opts_{dtype}", L, 4, 2, 64, 128, dtype, 851), cu, raw=True,
                 dt_softplus=True, dt_limit=(4e-3, 3e-2), zoh=True)


def test_varlen_mamba2_2p7b_packed_sampled():
    """The 2.7B layer's shape packed: 16384 tokens (8 x 2048) of 80 heads in
    sequences of 1 .. 4096 tokens; sampled heads against the oracle."""
    w = W.Workload("vl_2p7b_packed", 1, 16384, 80, 64, 1, 64, 256, "bf16", 1 / 8, 1e-3, 1e-1,
                   seed=860)
    cu = W.packed_cu_seqlens(w.seqlen, 4096, seed=861)
    check_varlen(w, cu, units=[0, 17, 41, 79])


def test_varlen_sequences_are_independent():
    """Changing one sequence's inputs changes nothing in the others."""
    ssd = _ssd()
    w = _w("vl_indep", 400, 4, 1, 64, 64, "bf16", 870)
    d = W.generate(w)
    g = {k: up(d[k]) for k in ("x", "dt", "A", "B", "C", "D")}
    cu_np = np.array([0, 70, 150, 151, 400], np.int32)
    cu = torch.from_numpy(cu_np).cuda()
    y1, s1 = ssd.forward_varlen(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], cu, chunk=64,
                                return_seq_states=True)
    x2 = g["x"].clone()
    x2[0, 70:150] = torch.randn_like(x2[0, 70:150].float()).to(x2.dtype)
    y2, s2 = ssd.forward_varlen(x2, g["dt"], g["A"], g["B"], g["C"], g["D"], cu, chunk=64,
                                return_seq_states=True)
    torch.cuda.synchronize()
    keep = torch.ones(400, dtype=torch.bool, device="cuda")
    keep[70:150] = False
    assert torch.equal(y1[0, keep], y2[0, keep])
    assert torch.equal(s1[[0, 2, 3]], s2[[0, 2, 3]]) and not torch.equal(s1[1], s2[1])


def test_varlen_errors():
    ssd = _ssd()
    x = torch.zeros((1, 10, 2, 64), dtype=torch.bfloat16, device="cuda")
    dt = torch.zeros((1, 10, 2), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros(2, dtype=torch.float32, device="cuda")
    B = torch.zeros((1, 10, 1, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):  # batch 2
        ssd.forward_varlen(torch.zeros((2, 10, 2, 64), dtype=torch.bfloat16, device="cuda"),
                           dt, A, B, B, None, torch.tensor([0, 10], dtype=torch.int32, device="cuda"))
    with pytest.raises(TypeError):  # int64 offsets
        ssd.forward_varlen(x, dt, A, B, B, None, torch.tensor([0, 10], device="cuda"))
    with pytest.raises(ValueError):  # no sequence
        ssd.forward_varlen(x, dt, A, B, B, None, torch.tensor([0], dtype=torch.int32, device="cuda"))


# ------------------- packed sequences on the single-pass kernel (bf16, N 64 / 128)
#
# With nheads a multiple of 8 the packed forward runs as the single-pass
# kernel with sequence masks (over several segments of the token axis): rows
# ignore the entering state and earlier sequences' tokens, the state resets
# where a sequence begins, and a sequence ending inside a 64-token block gets
# its state from the state entering the block and the block's own tokens.

def _plan(w):
    return _ssd().forward_plan(1, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate, w.chunk,
                               torch.bfloat16)


# boundaries on 64-token block starts (64, 128, 192, 1024) and ends (63, 191),
# inside blocks and at their 32-token half (160), an empty sequence, one-token
# sequences (at the start, 1999), sequences across the segments of the
# token axis (200 .. 700 .. 1024 .. 1500)
EXPLICIT_OP = [0, 1, 1, 9, 63, 64, 65, 128, 160, 191, 192, 200, 700, 701, 1024, 1500, 1999,
               2000]


@pytest.mark.parametrize("N", [64, 128])
def test_varlen_onepass_explicit_boundaries(N):
    w = _w(f"vl_op_explicit_N{N}", 2000, 8, 2, N, 256, "bf16", 880 + N)
    assert _plan(w) > 1
    check_varlen(w, EXPLICIT_OP)


@pytest.mark.parametrize("N", [64, 128, 256])
def test_varlen_onepass_length_mix(N):
    L = 3000
    cu = W.packed_cu_seqlens(L, 400, seed=890 + N)
    w = _w(f"vl_op_mix_N{N}", L, 16, 2, N, 128, "bf16", 891 + N)
    assert _plan(w) > 1
    check_varlen(w, cu)


def test_varlen_onepass_many_short_sequences():
    # every sequence shorter than 12 tokens: several ends in every block
    L = 1024
    cu = W.packed_cu_seqlens(L, 12, seed=900)
    w = _w("vl_op_short", L, 8, 1, 64, 256, "bf16", 901)
    assert cu.size > 100 and _plan(w) > 1
    check_varlen(w, cu)


def test_varlen_onepass_with_options():
    L = 1200
    cu = W.packed_cu_seqlens(L, 300, seed=910)
    w = _w("vl_op_opts", L, 8, 2, 128, 128, "bf16", 911)
    assert _plan(w) > 1
    check_varlen(w, cu, raw=True, dt_softplus=True, dt_limit=(4e-3, 3e-2), zoh=True)


@pytest.mark.parametrize("N", [64, 128])
def test_varlen_onepass_one_sequence_equals_forward(N):
    """One sequence: the masks select what the plain single-pass forward
    computes (several segments). The two kernels are separate compilations
    whose multiply-adds may fuse differently, so outputs agree to rounding:
    almost every y element identical, the rest within rel-L2 1e-4 (a
    hundredth of the bf16 tolerance), float32 states within 1e-5."""
    ssd = _ssd()
    w = _w(f"vl_op_single_N{N}", 1500, 8, 2, N, 256, "bf16", 920 + N)
    assert _plan(w) > 1
    d = W.generate(w)
    g = {k: up(d[k]) for k in ("x", "dt", "A", "B", "C", "D")}
    cu = torch.tensor([0, w.seqlen], dtype=torch.int32, device="cuda")
    y1, s1 = ssd.forward_varlen(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], cu,
                                chunk=w.chunk, return_seq_states=True)
    y2, s2 = ssd.forward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], chunk=w.chunk,
                         return_final_state=True)
    torch.cuda.synchronize()
    same = (y1 == y2).float().mean().item()
    ey, es = rel_l2(down(y1), down(y2)), rel_l2(down(s1[0]), down(s2[0]))
    print_case(f"   identical y: {same:.6f}, rel_l2 y {ey:.2e}, state {es:.2e}")
    assert same > 0.99 and ey < 1e-4 and es < 1e-5


def test_varlen_onepass_sequences_are_independent():
    """Changing one sequence's inputs changes nothing in the others."""
    ssd = _ssd()
    w = _w("vl_op_indep", 1000, 8, 1, 64, 64, "bf16", 930)
    d = W.generate(w)
    g = {k: up(d[k]) for k in ("x", "dt", "A", "B", "C", "D")}
    cu = torch.tensor([0, 70, 450, 451, 1000], dtype=torch.int32, device="cuda")
    assert _plan(w) > 1
    y1, s1 = ssd.forward_varlen(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], cu, chunk=64,
                                return_seq_states=True)
    x2 = g["x"].clone()
    x2[0, 70:450] = torch.randn_like(x2[0, 70:450].float()).to(x2.dtype)
    y2, s2 = ssd.forward_varlen(x2, g["dt"], g["A"], g["B"], g["C"], g["D"], cu, chunk=64,
                                return_seq_states=True)
    torch.cuda.synchronize()
    keep = torch.ones(1000, dtype=torch.bool, device="cuda")
    keep[70:450] = False
    assert torch.equal(y1[0, keep], y2[0, keep])
    assert torch.equal(s1[[0, 2, 3]], s2[[0, 2, 3]]) and not torch.equal(s1[1], s2[1])


def test_varlen_onepass_sequences_across_segments():
    # 8192 tokens of 16 heads at N 128 in sequences of up to 3000 tokens: the
    # token axis runs as many segments, most sequences span several of them
    L = 8192
    cu = W.packed_cu_seqlens(L, 3000, seed=940)
    w = _w("vl_op_across", L, 16, 2, 128, 256, "bf16", 941)
    S = _plan(w)
    print_case(f"   segments {S}, sequences {cu.size - 1}")
    assert S >= 8
    check_varlen(w, cu, units=[0, 5, 9, 15])
