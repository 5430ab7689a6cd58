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


ALL_PINS = [pin_duality, pin_cumsum, pin_lti_geometric, pin_single_token, pin_no_memory,
            pin_state_carry, pin_forward_vs_step, pin_linearity, pin_groups, pin_golden]
