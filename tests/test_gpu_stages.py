"""GPU parity of each forward stage on its own, plus properties of the whole
path that hold at any size: determinism, split-sequence continuation (the
fixed-size state carries everything), forward/decode duality and error paths.

Stage references come from the fp64 oracle: the within-chunk cumsum is its
definition; a chunk's own state is the recurrence run over that chunk alone
from a zero state; the state entering chunk c is the recurrence's state after
token cQ-1. C B^T tiles are decoded from their documented fragment layout and
compared with C_i . B_j computed in float64.
"""
import numpy as np
import pytest

import oracle
import ssd_workloads as W
from gpu_util import down, print_case, rel_l2, tol, up

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _ssd():
    import structured_state_space_ssd_amd as ssd
    return ssd


CASES = [
    W.small("st_bf16", 2, 3 * 128 + 45, 4, 64, 2, 64, 128, "bf16", seed=501, init_std=0.2),
    W.small("st_f32", 1, 2 * 64 + 10, 3, 64, 1, 32, 64, "f32", seed=502, init_std=0.2),
    W.small("st_n256", 1, 300, 2, 64, 1, 256, 128, "bf16", seed=503),
]


def _stages(w):
    ssd = _ssd()
    d = W.generate(w)
    g = {k: up(d[k]) for k in ("x", "dt", "A", "B", "C", "D")}
    init = up(d["init"])
    out = ssd.stages(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], chunk=w.chunk, init_state=init)
    torch.cuda.synchronize()
    return d, out


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_stage_chunk_cumsum(w):
    print_case(f"[stage cumsum] {w.name}")
    d, out = _stages(w)
    s = down(out["dA_cumsum"])[:, :, : w.seqlen]
    ref = oracle.chunk_cumsum(d["dt"].val, d["A"], w.chunk)
    # fp32 prefix sums of at most Q terms: relative error well below 1e-5
    assert rel_l2(s, ref) < 1e-5
    # the input weights without options: dt itself in float32, exact, zero past the end
    dl = down(out["delta"])
    Lp = w.nchunks * w.chunk
    want = np.zeros((w.batch, w.nheads, Lp))
    want[:, :, : w.seqlen] = d["dt"].val.astype(np.float64).transpose(0, 2, 1)
    assert np.array_equal(dl, want)


@pytest.mark.parametrize("zoh", [False, True])
@pytest.mark.parametrize("w", CASES[:2], ids=lambda w: w.name)
def test_stage_chunk_cumsum_options(w, zoh):
    """Stage 1 with bias + softplus + clamp (and the zero-order hold): s sums
    step * A over the preprocessed steps and delta holds each token's input
    weight, both against float64 numpy written from the definitions."""
    print_case(f"[stage cumsum options] {w.name} zoh={zoh}")
    ssd = _ssd()
    raw = W.generate_dt_raw(w)
    d = W.generate(w)
    sp = np.logaddexp(0.0, raw["dt"].val.astype(np.float64) + raw["dt_bias"])
    # clamp bounds at the 15th and 85th percentiles: both sides are hit
    lo, hi = (np.float32(np.quantile(sp, q)) for q in (0.15, 0.85))
    opts = ssd.options(dt_bias=up(raw["dt_bias"]), dt_softplus=True, dt_limit=(lo, hi), zoh=zoh)
    s, dl = ssd.chunk_cumsum(up(raw["dt"]), up(d["A"]), w.chunk, return_delta=True, opts=opts)
    torch.cuda.synchronize()
    A = d["A"].astype(np.float64)
    step = np.clip(sp, lo, hi)
    assert (step == lo).mean() > 0.1 and (step == hi).mean() > 0.1
    ref_s = oracle.chunk_cumsum(step, A, w.chunk)
    assert rel_l2(down(s)[:, :, : w.seqlen], ref_s) < 1e-5
    wt = np.expm1(step * A) / A if zoh else step
    Lp = w.nchunks * w.chunk
    want = np.zeros((w.batch, w.nheads, Lp))
    want[:, :, : w.seqlen] = wt.transpose(0, 2, 1)
    got = down(dl)
    assert np.all(got[:, :, w.seqlen:] == 0)
    assert np.allclose(got, want, rtol=5e-6, atol=0)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_stage_chunk_state(w):
    print_case(f"[stage chunk_state] {w.name}")
    d, out = _stages(w)
    st = down(out["states"])  # [Bt, nC, H, P, N]
    Bt, H, Q = w.batch, w.nheads, w.chunk
    for c in range(w.nchunks):
        sl = slice(c * Q, min((c + 1) * Q, w.seqlen))
        part = lambda a: np.ascontiguousarray(a[:, sl])
        _, s_ref, _ = oracle.forward(part(d["x"].val), part(d["dt"].val), d["A"], part(d["B"].val),
                                     part(d["C"].val), None, None)
        got = st[:, c].reshape(Bt * H, w.headdim, w.dstate)
        assert rel_l2(got, s_ref) < tol(w.dtype), (c, rel_l2(got, s_ref))


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_stage_state_passing(w):
    print_case(f"[stage state_passing] {w.name}")
    d, out = _stages(w)
    ci = down(out["chunk_init"])  # [Bt, nC, H, P, N] (operand type)
    Bt, H, Q = w.batch, w.nheads, w.chunk
    _, final, snaps = oracle.forward(d["x"].val, d["dt"].val, d["A"], d["B"].val, d["C"].val, None,
                                     d["init"], snap_every=Q)
    init = d["init"] if d["init"] is not None else np.zeros((Bt, H, w.headdim, w.dstate))
    for c in range(w.nchunks):
        ref = init.reshape(Bt * H, w.headdim, w.dstate) if c == 0 else snaps[:, c - 1]
        got = ci[:, c].reshape(Bt * H, w.headdim, w.dstate)
        assert rel_l2(got, ref) < tol(w.dtype), (c, rel_l2(got, ref))
    got_final = down(out["final_state"]).reshape(Bt * H, w.headdim, w.dstate)
    assert rel_l2(got_final, final) < tol(w.dtype)


def _decode_cb(cb_bytes, w, dtype_np):
    """Rebuild the causal C.B^T matrices [Bt, nC, G, Q, Q] from the fragment
    layout documented in include/ssd.h and chunk_cb.hip."""
    Q = w.chunk
    nt = Q // 16
    entries = (nt // 2) * (nt // 2 + 1)
    vals = cb_bytes.reshape(w.batch, w.nchunks, w.ngroups, entries, 64, 8)
    M = np.zeros((w.batch, w.nchunks, w.ngroups, Q, Q))
    e_idx = 0
    for it in range(nt):
        for jp in range(it // 2 + 1):
            for lane in range(64):
                g, r = lane // 16, lane % 16
                i = 16 * it + r
                for e in range(8):
                    j = 32 * jp + (4 * g + e if e < 4 else 16 + 4 * g + e - 4)
                    M[:, :, :, i, j] = vals[:, :, :, e_idx, lane, e]
            e_idx += 1
    return M


@pytest.mark.parametrize("w", [CASES[0], CASES[1]], ids=lambda w: w.name)
def test_stage_chunk_cb(w):
    print_case(f"[stage chunk_cb] {w.name}")
    d, out = _stages(w)
    raw = out["cb"].cpu()
    if w.dtype == "bf16":
        vals = raw.view(torch.bfloat16).float().numpy()
    else:
        vals = raw.view(torch.float32).numpy()
    M = _decode_cb(vals, w, None)
    Q = w.chunk
    B, C = d["B"].val.astype(np.float64), d["C"].val.astype(np.float64)
    for b in range(w.batch):
        for c in range(w.nchunks):
            sl = slice(c * Q, min((c + 1) * Q, w.seqlen))
            n = sl.stop - sl.start
            for g in range(w.ngroups):
                ref = C[b, sl, g] @ B[b, sl, g].T
                got = M[b, c, g, :n, :n]
                mask = np.tril(np.ones((n, n), bool))
                assert rel_l2(got[mask], ref[mask]) < tol(w.dtype)


# ---------------------------------------------------------------- properties

def test_deterministic_bitwise():
    ssd = _ssd()
    w = W.small("det", 2, 700, 8, 64, 2, 128, 256, "bf16", seed=510, init_std=0.1)
    d = W.generate(w)
    g = {k: up(d[k]) for k in ("x", "dt", "A", "B", "C", "D", "init")}
    y1, s1 = ssd.forward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], chunk=w.chunk,
                         init_state=g["init"], return_final_state=True)
    y2, s2 = ssd.forward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], chunk=w.chunk,
                         init_state=g["init"], return_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(s1, s2)


@pytest.mark.parametrize("k", [128, 300])
def test_split_sequence_continuation(k):
    """forward(x[:k]) -> final state -> forward(x[k:], init=state) reproduces
    forward(x); both halves checked against the oracle."""
    ssd = _ssd()
    w = W.small("split", 2, 640, 4, 64, 1, 64, 128, "bf16", seed=511)
    d = W.generate(w)
    g = {k_: up(d[k_]) for k_ in ("x", "dt", "A", "B", "C", "D")}
    sl = lambda t, s: t[:, s].contiguous()
    y1, s1 = ssd.forward(sl(g["x"], slice(0, k)), sl(g["dt"], slice(0, k)), g["A"],
                         sl(g["B"], slice(0, k)), sl(g["C"], slice(0, k)), g["D"], chunk=w.chunk,
                         return_final_state=True)
    y2, s2 = ssd.forward(sl(g["x"], slice(k, None)), sl(g["dt"], slice(k, None)), g["A"],
                         sl(g["B"], slice(k, None)), sl(g["C"], slice(k, None)), g["D"],
                         chunk=w.chunk, init_state=s1, return_final_state=True)
    torch.cuda.synchronize()
    y = np.concatenate([down(y1), down(y2)], axis=1)
    yo, so, _ = oracle.forward(d["x"].val, d["dt"].val, d["A"], d["B"].val, d["C"].val, d["D"])
    yo = yo.reshape(w.batch, w.nheads, w.seqlen, 64).transpose(0, 2, 1, 3)
    assert rel_l2(y, yo) < tol("bf16")
    assert rel_l2(down(s2).reshape(so.shape), so) < tol("bf16")


def test_forward_equals_decode_steps():
    """The chunked forward and L recurrent steps on the device agree (the
    'train with the matrix form, infer with the recurrence' duality)."""
    ssd = _ssd()
    w = W.small("dual", 2, 96, 4, 64, 2, 128, 64, "f32", seed=512, init_std=0.3)
    d = W.generate(w)
    g = {k: up(d[k]) for k in ("x", "dt", "A", "B", "C", "D", "init")}
    y, fs = ssd.forward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], chunk=w.chunk,
                        init_state=g["init"], return_final_state=True)
    state = g["init"].clone()
    ys = []
    for t in range(w.seqlen):
        ys.append(ssd.step(state, g["x"][:, t].contiguous(), g["dt"][:, t].contiguous(), g["A"],
                           g["B"][:, t].contiguous(), g["C"][:, t].contiguous(), g["D"]))
    torch.cuda.synchronize()
    yst = torch.stack(ys, dim=1)
    assert rel_l2(down(yst), down(y)) < 1e-4
    assert rel_l2(down(state), down(fs)) < 1e-4


def test_errors_raise_before_launch():
    ssd = _ssd()
    x = torch.zeros((1, 10, 3, 64), dtype=torch.bfloat16, device="cuda")
    dt = torch.zeros((1, 10, 3), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros(3, dtype=torch.float32, device="cuda")
    B = torch.zeros((1, 10, 2, 64), dtype=torch.bfloat16, device="cuda")  # 3 heads, 2 groups
    with pytest.raises(ssd.SSDError):
        ssd.forward(x, dt, A, B, B.clone(), chunk=64)
    B1 = torch.zeros((1, 10, 1, 40), dtype=torch.bfloat16, device="cuda")  # N not a multiple of 16
    with pytest.raises(ssd.SSDError):
        ssd.forward(x, dt, A, B1, B1.clone(), chunk=64)
    with pytest.raises(ssd.SSDError):
        ssd.forward(x, dt, A, B1[..., :32].contiguous(), B1[..., :32].contiguous(), chunk=96)
    B2 = torch.zeros((1, 10, 1, 272), dtype=torch.bfloat16, device="cuda")  # N above 256
    with pytest.raises(ssd.SSDError):
        ssd.forward(x, dt, A, B2, B2.clone(), chunk=64)
    with pytest.raises(TypeError):
        ssd.forward(x.half(), dt.half(), A, B1, B1, chunk=64)
