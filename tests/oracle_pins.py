"""Pins of the fp64 oracle to facts outside itself.

Each pin takes ``lib`` (None: the built oracle; a path: another build of the
oracle source, e.g. one with a planted mistake) and raises AssertionError when
the oracle disagrees with what the pages and the mathematics fix. The pins are
shared by the plain oracle tests and by the mutation test, which checks that a
planted mistake anywhere in the oracle trips at least one of them.
"""
import json
import math
import os

import numpy as np

import oracle
import ssd_workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _vals(w, seed=None):
    d = W.generate(w, seed)
    return {k: (v.val if isinstance(v, W.Tensor) else v) for k, v in d.items()}


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b.ravel())
    return np.linalg.norm((a - b).ravel()) / (den if den > 0 else 1.0)


def _units_to_bthp(y, Bt, H):
    U, L, P = y.shape
    return y.reshape(Bt, H, L, P).transpose(0, 2, 1, 3)


def pin_duality(lib=None):
    """P1: recurrence == quadratic (semiseparable) form on tiny random inputs.

    The SSD page ("Mamba 模型", section 4.1) writes the SSM as y = M x with the
    lower-triangular semiseparable M_ji = C_j^T A_{j:i} B_i; the "Mamba-2架构深度解析"
    page's section 2.2 lists this as the quadratic mode. Computed independently
    in numpy with exp of cumulative-sum differences.
    """
    cases = [
        W.small("p1a", 2, 23, 4, 6, 2, 5, 8, "f32", seed=11, init_std=0.3),
        W.small("p1b", 1, 40, 3, 4, 1, 7, 8, "f32", seed=12),
        W.small("p1c", 1, 17, 6, 3, 3, 4, 8, "f32", seed=13, init_std=1.0, dt_lo=0.05, dt_hi=2.0),
    ]
    for w in cases:
        v = _vals(w)
        y, st, _ = oracle.forward(v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], v["init"], lib=lib)
        yq, hq = oracle.quadratic(v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], v["init"])
        Bt, L, H, P = v["x"].shape
        assert _rel(_units_to_bthp(y, Bt, H), yq) < 1e-12, w.name
        assert _rel(st.reshape(Bt, H, P, -1), hq) < 1e-12, w.name


def pin_cumsum(lib=None):
    """P2: A = 0, dt = 1, B = C = e_0 makes the state a running sum of x.

    exp(0) = 1 (no decay), so y_t = sum_{j<=t} x_j + D x_t exactly.
    """
    rng = np.random.default_rng(5)
    Bt, L, H, P, N = 1, 50, 2, 3, 4
    x = rng.integers(-8, 9, size=(Bt, L, H, P)).astype(np.float32)
    dt = np.ones((Bt, L, H), np.float32)
    A = np.zeros(H, np.float32)
    B = np.zeros((Bt, L, 1, N), np.float32)
    B[..., 0] = 1
    C = B.copy()
    D = np.array([0.5, -2.0], np.float32)
    y, st, _ = oracle.forward(x, dt, A, B, C, D, lib=lib)
    expect = np.cumsum(x, axis=1) + D[None, None, :, None] * x
    assert np.array_equal(_units_to_bthp(y, Bt, H), expect)
    assert np.array_equal(st[:, :, 0], np.cumsum(x, axis=1)[0, -1])
    assert not st[:, :, 1:].any()


def pin_lti_geometric(lib=None):
    """P3: time-invariant case (constant dt, B, C) gives the convolution kernel
    K_k = C Abar^k Bbar ("Mamba 模型", section 2.3.2; "深挖-Mamba", core
    concept 2): y_t = dt (C.B) sum_{j<=t} alpha^{t-j} x_j + D x_t, and for a
    constant x the geometric series dt (C.B) x (1 - alpha^{t+1}) / (1 - alpha).
    """
    rng = np.random.default_rng(6)
    Bt, L, H, P, N = 1, 64, 2, 4, 8
    dtv = np.array([0.3, 0.05], np.float32)
    A = np.array([-1.5, -4.0], np.float32)
    D = np.array([0.25, -0.75], np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    c = rng.standard_normal(N).astype(np.float32)
    dt = np.broadcast_to(dtv, (Bt, L, H)).copy()
    B = np.broadcast_to(b, (Bt, L, 1, N)).copy()
    C = np.broadcast_to(c, (Bt, L, 1, N)).copy()
    cb = float(np.dot(c.astype(np.float64), b.astype(np.float64)))
    # random x: explicit convolution with the kernel dt (C.B) alpha^k
    x = rng.standard_normal((Bt, L, H, P)).astype(np.float32)
    y, _, _ = oracle.forward(x, dt, A, B, C, D, lib=lib)
    y = _units_to_bthp(y, Bt, H)
    for h in range(H):
        alpha = math.exp(float(dtv[h]) * float(A[h]))
        k = float(dtv[h]) * cb * alpha ** np.arange(L)
        conv = np.array([[np.dot(k[: t + 1][::-1], x[0, : t + 1, h, p].astype(np.float64))
                          for p in range(P)] for t in range(L)])
        expect = conv + float(D[h]) * x[0, :, h, :].astype(np.float64)
        assert _rel(y[0, :, h, :], expect) < 1e-12
    # constant x: closed-form geometric sum
    xc = np.ones((Bt, L, H, P), np.float32) * np.float32(1.5)
    y, _, _ = oracle.forward(xc, dt, A, B, C, D, lib=lib)
    y = _units_to_bthp(y, Bt, H)
    t = np.arange(L)
    for h in range(H):
        alpha = math.exp(float(dtv[h]) * float(A[h]))
        expect = float(dtv[h]) * cb * 1.5 * (1 - alpha ** (t + 1)) / (1 - alpha) + float(D[h]) * 1.5
        assert np.max(np.abs(y[0, :, h, 0] - expect)) < 1e-12 * max(1.0, np.max(np.abs(expect)))


def pin_single_token(lib=None):
    """P4: L = 1 from a zero state: y = dt (C.B) x + D x, state = dt x B^T."""
    w = W.small("p4", 3, 1, 4, 5, 2, 6, 8, "f32", seed=14)
    v = _vals(w)
    y, st, _ = oracle.forward(v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], lib=lib)
    x, dt, B, C, D = (v[k].astype(np.float64) for k in ("x", "dt", "B", "C", "D"))
    Bt, H, G = 3, 4, 2
    for b in range(Bt):
        for h in range(H):
            g = h // (H // G)
            u = b * H + h
            cb = np.dot(C[b, 0, g], B[b, 0, g])
            assert np.allclose(y[u, 0], dt[b, 0, h] * cb * x[b, 0, h] + D[h] * x[b, 0, h], rtol=1e-13, atol=1e-15)
            assert np.allclose(st[u], dt[b, 0, h] * np.outer(x[b, 0, h], B[b, 0, g]), rtol=1e-13, atol=1e-15)


def pin_no_memory(lib=None):
    """P5: A -> -inf makes exp(dt A) = 0, so each token sees only itself."""
    w = W.small("p5", 2, 12, 2, 4, 1, 5, 8, "f32", seed=15)
    v = _vals(w)
    A = np.full(2, -1e6, np.float32)
    y, _, _ = oracle.forward(v["x"], v["dt"], A, v["B"], v["C"], v["D"], lib=lib)
    x, dt, B, C, D = (v[k].astype(np.float64) for k in ("x", "dt", "B", "C", "D"))
    cb = np.einsum("bln,bln->bl", C[:, :, 0], B[:, :, 0])
    expect = dt[..., None] * cb[:, :, None, None] * x + D[None, None, :, None] * x
    assert _rel(_units_to_bthp(y, 2, 2), expect) < 1e-13


def pin_state_carry(lib=None):
    """P7: the fixed-size state carries the whole past ("深挖-Mamba", comparison
    table: no KV cache, only the hidden state): running [0, k) then [k, L) from
    the carried state equals running [0, L). Also checks the state snapshots."""
    w = W.small("p7", 2, 30, 3, 4, 1, 6, 8, "f32", seed=16, init_std=0.2)
    v = _vals(w)
    k = 13
    y, st, snaps = oracle.forward(v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], v["init"],
                                  snap_every=k, lib=lib)
    sl = lambda a, s: np.ascontiguousarray(a[:, s])
    y1, st1, _ = oracle.forward(sl(v["x"], slice(0, k)), sl(v["dt"], slice(0, k)), v["A"],
                                sl(v["B"], slice(0, k)), sl(v["C"], slice(0, k)), v["D"], v["init"], lib=lib)
    y2, st2, _ = oracle.forward(sl(v["x"], slice(k, None)), sl(v["dt"], slice(k, None)), v["A"],
                                sl(v["B"], slice(k, None)), sl(v["C"], slice(k, None)), v["D"],
                                st1.reshape(2, 3, 4, 6), lib=lib)
    assert np.max(np.abs(np.concatenate([y1, y2], axis=1) - y)) < 1e-13
    assert np.max(np.abs(st2 - st)) < 1e-13
    assert snaps.shape[1] == 30 // k
    assert np.max(np.abs(snaps[:, 0] - st1)) < 1e-13


def pin_forward_vs_step(lib=None):
    """P8: L recurrent steps equal one forward ("深挖-Mamba", Mamba-2: train
    with the matrix form, infer with the recurrence)."""
    w = W.small("p8", 2, 9, 4, 3, 2, 5, 8, "f32", seed=17, init_std=0.5)
    v = _vals(w)
    y, st, _ = oracle.forward(v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], v["init"], lib=lib)
    state = np.ascontiguousarray(v["init"].reshape(8, 3, 5).astype(np.float64))
    for t in range(9):
        ys = oracle.step(state, v["x"][:, t], v["dt"][:, t], v["A"], v["B"][:, t], v["C"][:, t],
                         v["D"], lib=lib)
        assert np.max(np.abs(ys - y[:, t])) < 1e-13
    assert np.max(np.abs(state - st)) < 1e-13


def pin_linearity(lib=None):
    """P9: the SSM is a linear system in x and in the initial state."""
    w = W.small("p9", 1, 20, 2, 4, 1, 5, 8, "f32", seed=18, init_std=1.0)
    v = _vals(w)
    rng = np.random.default_rng(9)
    # dyadic inputs so that x1 + x2 is exact in float32
    x1 = (rng.integers(-64, 65, size=v["x"].shape) / 16).astype(np.float32)
    x2 = rng.integers(-4, 5, size=v["x"].shape).astype(np.float32)
    args = (v["dt"], v["A"], v["B"], v["C"], v["D"])
    ya, _, _ = oracle.forward(x1, *args, lib=lib)
    yb, _, _ = oracle.forward(x2, *args, lib=lib)
    yab, _, _ = oracle.forward(x1 + x2, *args, lib=lib)
    assert _rel(yab, ya + yb) < 1e-12
    zero = np.zeros_like(v["x"])
    y1, s1, _ = oracle.forward(zero, *args, init=v["init"], lib=lib)
    y3, s3, _ = oracle.forward(zero, *args, init=3.0 * v["init"].astype(np.float64), lib=lib)
    assert _rel(y3, 3 * y1) < 1e-13 and _rel(s3, 3 * s1) < 1e-13
    assert np.abs(y1).max() > 0


def pin_groups(lib=None):
    """P10 and the head-to-group map: B/C are shared by H/G consecutive heads
    ("Draft:Mamba2" and "Mamba 模型" section 4.3: grouped-value heads).
    (a) G = H with replicated B, C equals G = 1; (b) with H = 4, G = 2, zeroing
    group 1's B leaves heads 2, 3 with only D x and heads 0, 1 untouched."""
    w = W.small("p10", 2, 15, 4, 3, 1, 5, 8, "f32", seed=19)
    v = _vals(w)
    y1, s1, _ = oracle.forward(v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], lib=lib)
    Brep = np.repeat(v["B"], 4, axis=2)
    Crep = np.repeat(v["C"], 4, axis=2)
    y4, s4, _ = oracle.forward(v["x"], v["dt"], v["A"], Brep, Crep, v["D"], lib=lib)
    assert np.array_equal(y1, y4) and np.array_equal(s1, s4)
    rng = np.random.default_rng(10)
    B2 = rng.standard_normal((2, 15, 2, 5)).astype(np.float32)
    C2 = rng.standard_normal((2, 15, 2, 5)).astype(np.float32)
    B2[:, :, 0] = v["B"][:, :, 0]
    C2[:, :, 0] = v["C"][:, :, 0]
    B2z = B2.copy()
    B2z[:, :, 1] = 0
    yg, _, _ = oracle.forward(v["x"], v["dt"], v["A"], B2z, C2, v["D"], lib=lib)
    yg = _units_to_bthp(yg, 2, 4)
    y1b = _units_to_bthp(y1, 2, 4)
    dx = v["D"][None, None, :, None].astype(np.float64) * v["x"]
    assert np.array_equal(yg[:, :, 2:], dx[:, :, 2:])
    assert np.array_equal(yg[:, :, :2], y1b[:, :, :2])


def pin_golden(lib=None):
    """Hand-worked three-token example (tests/golden/worked_example.json)."""
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    x = np.array(g["x"], np.float32)[None, :, None, :]
    dt = np.array(g["dt"], np.float32)[None, :, None]
    B = np.array(g["B"], np.float32)[None, :, None, :]
    C = np.array(g["C"], np.float32)[None, :, None, :]
    A = np.array([-math.log(2.0)], np.float32)
    D = np.array([g["D"]], np.float32)
    y, st, _ = oracle.forward(x, dt, A, B, C, D, lib=lib)
    assert np.allclose(y[0], np.array(g["y"]), rtol=1e-7, atol=1e-7)
    assert np.allclose(st[0], np.array(g["final_state"]), rtol=1e-7, atol=1e-7)


def _dyadic(rng, shape, lo, hi, denom):
    """float32 values k / denom, k uniform in [lo*denom, hi*denom]: sums of two
    such values are exact in float32."""
    return (rng.integers(int(lo * denom), int(hi * denom) + 1, size=shape) / denom).astype(np.float32)


def pin_dt_bias(lib=None):
    """P11: the per-head bias is added to the raw step size before anything
    else (the constant term of the step-size projection of the
    "从Transformer到Mamba" tutorial, section 3.2). With dyadic values the
    sum is exact, so forward(dt, bias) must equal forward(dt + bias)
    bit for bit, for the forward and for the recurrent step."""
    w = W.small("p11", 2, 13, 4, 3, 2, 5, 8, "f32", seed=21, init_std=0.4)
    v = _vals(w)
    rng = np.random.default_rng(21)
    raw = _dyadic(rng, v["dt"].shape, -0.1, 0.1, 256)
    bias = _dyadic(rng, (4,), 0.11, 0.4, 256)
    shifted = (raw + bias[None, None, :]).astype(np.float32)
    assert np.array_equal(shifted.astype(np.float64), raw.astype(np.float64) + bias)
    args = (v["A"], v["B"], v["C"], v["D"], v["init"])
    y0, s0, _ = oracle.forward(v["x"], raw, *args, dt_bias=bias, lib=lib)
    y1, s1, _ = oracle.forward(v["x"], shifted, *args, lib=lib)
    assert np.array_equal(y0, y1) and np.array_equal(s0, s1)
    st_a = np.ascontiguousarray(v["init"].reshape(8, 3, 5).astype(np.float64))
    st_b = st_a.copy()
    ya = oracle.step(st_a, v["x"][:, 0], raw[:, 0], v["A"], v["B"][:, 0], v["C"][:, 0], v["D"],
                     dt_bias=bias, lib=lib)
    yb = oracle.step(st_b, v["x"][:, 0], shifted[:, 0], v["A"], v["B"][:, 0], v["C"][:, 0], v["D"],
                     lib=lib)
    assert np.array_equal(ya, yb) and np.array_equal(st_a, st_b)


def pin_softplus_and_clamp(lib=None):
    """P12: softplus (tutorial section 3.2) is log(1 + e^v), checked against
    numpy's logaddexp(0, v) over raw values from -9 to 40; the clamp (the
    step-size range of the tutorial's section 8.2) is numpy's clip and comes
    after softplus, and the bias comes before both."""
    w = W.small("p12", 2, 17, 4, 3, 2, 5, 8, "f32", seed=22, init_std=0.4)
    v = _vals(w)
    rng = np.random.default_rng(22)
    raw = _dyadic(rng, v["dt"].shape, -9.0, 2.0, 64)
    raw[0, 3, :] = [20.0, 40.0, -20.0, 0.0]
    args = (v["A"], v["B"], v["C"], v["D"], v["init"])
    sp = np.logaddexp(0.0, raw.astype(np.float64)).astype(np.float32)
    y0, s0, _ = oracle.forward(v["x"], raw, *args, dt_softplus=True, lib=lib)
    y1, s1, _ = oracle.forward(v["x"], sp, *args, lib=lib)
    assert _rel(y0, y1) < 2e-6 and _rel(s0, s1) < 2e-6
    # clamp alone: exact, bounds are float32 values
    lo, hi = 0.0625, 0.25
    pos = _dyadic(rng, v["dt"].shape, 0.0, 0.5, 1024)
    y0, s0, _ = oracle.forward(v["x"], pos, *args, dt_limit=(lo, hi), lib=lib)
    y1, s1, _ = oracle.forward(v["x"], np.clip(pos, lo, hi), *args, lib=lib)
    assert np.array_equal(y0, y1) and np.array_equal(s0, s1)
    # the whole chain: clip(softplus(raw + bias)), bounds hit on both sides
    bias = np.array([-4.0, -2.5, -1.0, 0.5], np.float32)
    lo, hi = 0.02, 0.3
    ref = np.clip(np.logaddexp(0.0, raw.astype(np.float64) + bias), lo, hi)
    assert (ref == lo).mean() > 0.1 and (ref == hi).mean() > 0.1
    y0, s0, _ = oracle.forward(v["x"], raw, *args, dt_bias=bias, dt_softplus=True,
                               dt_limit=(lo, hi), lib=lib)
    y1, s1, _ = oracle.forward(v["x"], ref.astype(np.float32), *args, lib=lib)
    assert _rel(y0, y1) < 2e-6 and _rel(s0, s1) < 2e-6


def _ode_zoh_reference(x, dt, A, B, C, D, init):
    """Integrate dh/dtau = A h + x_t B_t^T over [0, dt_t] per token with the
    input held constant on each interval (zero-order hold), then read
    y_t = C_t . h + D x_t. One batch, one group; float64 lists of arrays."""
    from scipy.integrate import solve_ivp
    L, H, P = x.shape
    N = B.shape[-1]
    y = np.zeros((L, H, P))
    hf = np.zeros((H, P, N))
    for h in range(H):
        state = np.array(init[h], np.float64).ravel()
        for t in range(L):
            drive = np.outer(x[t, h], B[t]).ravel()
            sol = solve_ivp(lambda _tau, s, a=float(A[h]), u=drive: a * s + u,
                            (0.0, float(dt[t, h])), state, method="DOP853",
                            rtol=1e-12, atol=1e-14)
            state = sol.y[:, -1]
            y[t, h] = state.reshape(P, N) @ C[t] + D[h] * x[t, h]
        hf[h] = state.reshape(P, N)
    return y, hf


def pin_zoh_ode(lib=None):
    """P13: with zoh, each token advances the state by the exact solution of
    the continuous SSM dh/dt = A h + B u (tutorial section 2.1) over a step of
    length dt with the input held constant: the zero-order hold of the
    tutorial's section 2.2 and "Mamba 模型" section 2.3.1. The reference is a
    numerical ODE solve, independent of any closed form."""
    w = W.small("p13", 1, 7, 2, 2, 1, 3, 8, "f32", seed=23, init_std=0.5, dt_lo=0.05, dt_hi=1.5)
    v = _vals(w)
    y, st, _ = oracle.forward(v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], v["init"],
                              zoh=True, lib=lib)
    f64 = lambda a: np.asarray(a, np.float64)
    yr, hr = _ode_zoh_reference(f64(v["x"][0]), f64(v["dt"][0]), f64(v["A"]), f64(v["B"][0, :, 0]),
                                f64(v["C"][0, :, 0]), f64(v["D"]), f64(v["init"][0]))
    assert _rel(_units_to_bthp(y, 1, 2)[0], yr) < 1e-9
    assert _rel(st.reshape(2, 2, 3), hr) < 1e-9


def pin_zoh_forms(lib=None):
    """P14: (a) the zoh weight (exp(dt A) - 1) / A tends to dt as A -> 0, and
    A = 0 gives the Euler weight exactly; (b) on grouped multi-head inputs
    with an initial state, the zoh recurrence equals the quadratic form with
    input weights expm1(dt A) / A (numpy), and differs from Euler."""
    w = W.small("p14", 2, 21, 4, 3, 2, 5, 8, "f32", seed=24, init_std=0.3, dt_lo=0.02, dt_hi=1.0)
    v = _vals(w)
    x, dt, B, C, D, init = v["x"], v["dt"], v["B"], v["C"], v["D"], v["init"]
    zero_a = np.zeros(4, np.float32)
    ye, se, _ = oracle.forward(x, dt, zero_a, B, C, D, init, lib=lib)
    yz, sz, _ = oracle.forward(x, dt, zero_a, B, C, D, init, zoh=True, lib=lib)
    assert np.array_equal(ye, yz) and np.array_equal(se, sz)
    tiny_a = np.full(4, -1e-9, np.float32)
    ye, se, _ = oracle.forward(x, dt, tiny_a, B, C, D, init, lib=lib)
    yz, sz, _ = oracle.forward(x, dt, tiny_a, B, C, D, init, zoh=True, lib=lib)
    assert _rel(yz, ye) < 1e-8 and _rel(sz, se) < 1e-8
    A = v["A"]
    yz, sz, _ = oracle.forward(x, dt, A, B, C, D, init, zoh=True, lib=lib)
    wts = np.expm1(dt.astype(np.float64) * A) / A.astype(np.float64)
    yq, hq = oracle.quadratic(x, dt, A, B, C, D, init, weights=wts)
    assert _rel(_units_to_bthp(yz, 2, 4), yq) < 1e-11
    assert _rel(sz.reshape(2, 4, 3, 5), hq) < 1e-11
    ye, _, _ = oracle.forward(x, dt, A, B, C, D, init, lib=lib)
    assert _rel(yz, ye) > 1e-3


def pin_step_with_options(lib=None):
    """P15: with every option on, L recurrent steps still equal one forward
    (the same preprocessing and input weight on both paths)."""
    w = W.small("p15", 2, 9, 4, 3, 2, 5, 8, "f32", seed=25, init_std=0.5)
    v = _vals(w)
    rng = np.random.default_rng(25)
    raw = _dyadic(rng, v["dt"].shape, -4.0, 1.0, 64)
    opts = dict(dt_bias=np.array([-1.0, 0.5, -2.0, 0.0], np.float32), dt_softplus=True,
                dt_limit=(0.05, 0.9), zoh=True)
    y, st, _ = oracle.forward(v["x"], raw, v["A"], v["B"], v["C"], v["D"], v["init"], lib=lib,
                              **opts)
    state = np.ascontiguousarray(v["init"].reshape(8, 3, 5).astype(np.float64))
    for t in range(9):
        ys = oracle.step(state, v["x"][:, t], raw[:, t], v["A"], v["B"][:, t], v["C"][:, t],
                         v["D"], lib=lib, **opts)
        assert np.max(np.abs(ys - y[:, t])) < 1e-13
    assert np.max(np.abs(state - st)) < 1e-13


def pin_varlen(lib=None):
    """P16: packed variable-length sequences ("Mamba-2架构深度解析" section 5,
    dynamic packing of variable-length sequences) are independent sequences:
    the packed run equals separate runs of each slice from the zero state,
    bit for bit, and the numpy quadratic form of each slice; every sequence's
    final state is the separate run's final state; an empty sequence's final
    state is zero; one sequence is the plain forward. Checked with and without
    the step-size options."""
    rng = np.random.default_rng(26)
    L, H, P, G, N = 41, 4, 3, 2, 5
    x = rng.standard_normal((1, L, H, P)).astype(np.float32)
    B = (rng.standard_normal((1, L, G, N)) / 2).astype(np.float32)
    C = (rng.standard_normal((1, L, G, N)) / 2).astype(np.float32)
    dt = np.exp(rng.uniform(np.log(0.05), np.log(0.8), (1, L, H))).astype(np.float32)
    A = -np.exp(rng.uniform(0.0, np.log(4.0), H)).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    raw = _dyadic(rng, (1, L, H), -3.0, 1.0, 64)
    bias = np.array([-1.0, 0.5, -2.0, 0.0], np.float32)
    # lengths 1, 0 (empty), 7, 1, 12, 0, 20: ends and starts next to each other
    cu = np.array([0, 1, 1, 8, 9, 21, 21, 41], np.int32)
    for opts, dts in ((dict(), dt), (dict(dt_bias=bias, dt_softplus=True, dt_limit=(0.05, 0.9),
                                         zoh=True), raw)):
        y, st = oracle.forward_varlen(x, dts, A, B, C, D, cu, lib=lib, **opts)
        assert y.shape == (H, L, P) and st.shape == (H, 7, P, N)
        for k in range(7):
            a, e = int(cu[k]), int(cu[k + 1])
            if a == e:
                assert np.all(st[:, k] == 0)
                continue
            sl = lambda t: np.ascontiguousarray(t[:, a:e])
            ys, ss, _ = oracle.forward(sl(x), sl(dts), A, sl(B), sl(C), D, lib=lib, **opts)
            assert np.array_equal(y[:, a:e], ys) and np.array_equal(st[:, k], ss)
            if not opts:
                yq, hq = oracle.quadratic(sl(x), sl(dts), A, sl(B), sl(C), D)
                assert _rel(_units_to_bthp(np.ascontiguousarray(y[:, a:e]), 1, H), yq) < 1e-12
                assert _rel(st[:, k], hq[0]) < 1e-12
    y1, st1 = oracle.forward_varlen(x, dt, A, B, C, D, np.array([0, L], np.int32), lib=lib)
    yf, sf, _ = oracle.forward(x, dt, A, B, C, D, lib=lib)
    assert np.array_equal(y1, yf) and np.array_equal(st1[:, 0], sf)


def _loss(x, dt, A, B, C, D, init, dy, dfinal, lib, **opts):
    """sum(dy * y) + sum(dfinal * final state) of the forward oracle, float64."""
    y, st, _ = oracle.forward(x, dt, A, B, C, D, init, lib=lib, **opts)
    Bt, L, H, P = x.shape
    y = y.reshape(Bt, H, L, P).transpose(0, 2, 1, 3)
    return float((y * dy).sum() + (st.reshape(dfinal.shape) * dfinal).sum())


def pin_backward_finite_differences(lib=None):
    """P17: every gradient of the backward oracle is the derivative of the
    (pinned) forward oracle: <dZ, V> equals the central difference
    (loss(Z + eps V) - loss(Z - eps V)) / (2 eps) for random directions V, with
    dyadic inputs so that Z +- eps V is exact in float32. The loss is
    sum(dy * y) + sum(dfinal * final state). Checked without options and with
    bias + softplus + clamp (bounds hit) + zero-order hold."""
    rng = np.random.default_rng(27)
    Bt, L, H, P, G, N = 2, 19, 4, 3, 2, 5
    dyad = lambda shape, lo, hi, den: _dyadic(rng, shape, lo, hi, den)
    base = dict(x=dyad((Bt, L, H, P), -2, 2, 16), B=dyad((Bt, L, G, N), -1, 1, 32),
                C=dyad((Bt, L, G, N), -1, 1, 32), A=-dyad((H,), 0.5, 4, 64), D=dyad((H,), -1, 1, 16),
                init=dyad((Bt, H, P, N), -1, 1, 8).astype(np.float64))
    dy = rng.standard_normal((Bt, L, H, P)).astype(np.float32)
    dfinal = rng.standard_normal((Bt, H, P, N))
    dts = dyad((Bt, L, H), 0.01, 0.3, 4096)
    raw = dyad((Bt, L, H), -4.0, 1.0, 4096)
    bias = np.array([-1.0, 0.25, -2.0, 0.0], np.float32)
    lo, hi = 0.05, 0.6
    for _ in range(20):  # keep every step away from the clamp's kinks
        sp = np.logaddexp(0.0, raw.astype(np.float64) + bias)
        near = np.minimum(np.abs(sp - lo), np.abs(sp - hi)) <= 1e-3
        if not near.any():
            break
        raw[near] += np.float32(1.0 / 32)
    assert not near.any()
    assert (sp < lo).mean() > 0.05 and (sp > hi).mean() > 0.02
    cases = [(dts, {}), (raw, dict(dt_bias=bias, dt_softplus=True, dt_limit=(lo, hi), zoh=True))]
    for dt, opts in cases:
        args = dict(base, dt=dt)
        grads = oracle.backward(args["x"], dt, args["A"], args["B"], args["C"], args["D"],
                                args["init"], dy, dfinal, lib=lib, **opts)
        steps = dict(x=2.0 ** -8, dt=2.0 ** -16, A=2.0 ** -14, B=2.0 ** -8, C=2.0 ** -8,
                     D=2.0 ** -8, init=2.0 ** -8)
        for name, eps in steps.items():
            V = rng.integers(-1, 2, size=args[name].shape).astype(np.float64)
            plus, minus = dict(args), dict(args)
            dtype = np.float64 if name == "init" else np.float32
            plus[name] = (args[name] + eps * V).astype(dtype)
            minus[name] = (args[name] - eps * V).astype(dtype)
            assert np.array_equal(plus[name].astype(np.float64) - args[name], eps * V)
            fd = (_loss(dy=dy, dfinal=dfinal, lib=lib, **plus, **opts) -
                  _loss(dy=dy, dfinal=dfinal, lib=lib, **minus, **opts)) / (2 * eps)
            an = float((grads["dinit" if name == "init" else "d" + name] * V).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, bool(opts), fd, an)
        if opts:  # the bias enters like a shift of every raw dt of its head
            eps = 2.0 ** -16
            V = rng.integers(-1, 2, size=H).astype(np.float64)
            bp = (bias + eps * V).astype(np.float32)
            bm = (bias - eps * V).astype(np.float32)
            o2 = dict(opts)
            fd = (_loss(dy=dy, dfinal=dfinal, lib=lib, **args, **dict(o2, dt_bias=bp)) -
                  _loss(dy=dy, dfinal=dfinal, lib=lib, **args, **dict(o2, dt_bias=bm))) / (2 * eps)
            an = float((grads["dbias"] * V).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), ("bias", fd, an)


def pin_backward_zoh_small_decay(lib=None):
    """P18: the zero-order-hold weight's derivative with respect to A where
    |dt A| is small (below 1e-3: the backward oracle's series form of
    (z e^z - expm1(z)) / A^2, whose closed form cancels there), checked like
    P17 against central differences of the pinned forward oracle. The heads'
    A are tiny dyadic values, so the weight w = expm1(dt A)/A is close to dt
    and its A-derivative is about dt^2/2 (1 + 2 z / 3): the step eps in A is
    small enough that the difference quotient resolves the z-term."""
    rng = np.random.default_rng(31)
    Bt, L, H, P, G, N = 1, 23, 3, 4, 1, 6
    dyad = lambda shape, lo, hi, den: _dyadic(rng, shape, lo, hi, den)
    args = dict(x=dyad((Bt, L, H, P), -2, 2, 16), B=dyad((Bt, L, G, N), -1, 1, 32),
                C=dyad((Bt, L, G, N), -1, 1, 32), D=dyad((H,), -1, 1, 16),
                init=dyad((Bt, H, P, N), -1, 1, 8).astype(np.float64),
                A=-np.array([2.0 ** -12 * 3, 2.0 ** -11 * 3, 2.0 ** -10 * 3], np.float32),
                dt=dyad((Bt, L, H), 0.02, 0.3, 4096))
    z = np.abs(args["dt"].astype(np.float64) * args["A"].astype(np.float64))
    assert z.max() < 1e-3 and (z > 3e-4).mean() > 0.15  # the series branch, with a z-term that shows
    dy = rng.standard_normal((Bt, L, H, P)).astype(np.float32)
    dfinal = rng.standard_normal((Bt, H, P, N))
    opts = dict(zoh=True)
    grads = oracle.backward(args["x"], args["dt"], args["A"], args["B"], args["C"], args["D"],
                            args["init"], dy, dfinal, lib=lib, **opts)
    for h in range(H):  # one head at a time: each dA[h] is checked on its own
        eps = 2.0 ** -20
        plus, minus = dict(args), dict(args)
        plus["A"] = args["A"].copy()
        minus["A"] = args["A"].copy()
        plus["A"][h] += np.float32(eps)
        minus["A"][h] -= np.float32(eps)
        assert plus["A"][h] - args["A"][h] == eps and args["A"][h] - minus["A"][h] == eps
        fd = (_loss(dy=dy, dfinal=dfinal, lib=lib, **plus, **opts) -
              _loss(dy=dy, dfinal=dfinal, lib=lib, **minus, **opts)) / (2 * eps)
        an = float(grads["dA"][h])
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (h, fd, an)


ALL_PINS = [pin_duality, pin_cumsum, pin_lti_geometric, pin_single_token, pin_no_memory,
            pin_state_carry, pin_forward_vs_step, pin_linearity, pin_groups, pin_golden,
            pin_dt_bias, pin_softplus_and_clamp, pin_zoh_ode, pin_zoh_forms,
            pin_step_with_options, pin_varlen, pin_backward_finite_differences,
            pin_backward_zoh_small_decay]
