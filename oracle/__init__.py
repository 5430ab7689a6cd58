"""fp64 CPU oracle for the SSD layer: TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. It shares no code with the HIP library and never imports it.

Contents
--------
* ``forward`` / ``step``: the token-by-token recurrence in C (``ssd_oracle.c``),
  fp64, threads over independent (batch, head) units.
* ``quadratic``: the dual "attention-like" form written out in numpy,
  y = (L o C B^T)(dt o x) + D x with L_ij = exp(sum_{k=j+1..i} dt_k A), the
  semiseparable matrix of the "Mamba 模型" page, section 4.1 (SSD), and the
  quadratic mode of the "Mamba-2架构深度解析" page's section 2.2 table. It is
  an independent O(L^2) computation used to pin the recurrence.
* ``chunk_cumsum``: the within-chunk inclusive prefix sum of dt*A, the first
  step of the block decomposition ("Mamba 模型", section 4.1).
* ``backward``: reverse-mode gradients of the forward (adjoint recurrence of
  the state, in fp64, with the states recomputed from checkpoints), with the
  same options.
* ``forward_varlen``: packed variable-length sequences (the dynamic sequence
  packing of the "Mamba-2架构深度解析" page, section 5): the recurrence with the
  state reset to zero where each sequence begins, and every sequence's final
  state.

Options (``forward``, ``step``): ``dt_bias`` [H] is added to the raw dt,
``dt_softplus`` applies log(1 + e^v) (the "从Transformer到Mamba" tutorial,
section 3.2, makes the step size positive this way), ``dt_limit = (lo, hi)``
clamps the result (the tutorial's section 8.2 adjusts the step-size range),
and ``zoh`` replaces the Euler input weight dt by the zero-order-hold weight
(exp(dt A) - 1) / A (tutorial section 2.2; "Mamba 模型" section 2.3.1).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssd_oracle.so")
SRC_PATH = os.path.join(_HERE, "ssd_oracle.c")

# Portable x86-64 level so the library built in one container runs on another
# host; plain IEEE double arithmetic (no fast-math, no FMA contraction).
CFLAGS = ["-O2", "-march=x86-64-v2", "-ffp-contract=off", "-fno-fast-math",
          "-std=c11", "-fPIC", "-shared", "-pthread"]


def build(force: bool = True, src: str = SRC_PATH, out: str = LIB_PATH) -> str:
    """Compile the oracle library with gcc; returns its path."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.run(["gcc", *CFLAGS, src, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, out)
    return out


_libs = {}


class _Opts(ctypes.Structure):
    _fields_ = [("dt_bias", ctypes.c_void_p), ("dt_softplus", ctypes.c_int),
                ("dt_clamp", ctypes.c_int), ("dt_min", ctypes.c_double),
                ("dt_max", ctypes.c_double), ("zoh", ctypes.c_int)]


def _opts(H, dt_bias, dt_softplus, dt_limit, zoh):
    """(struct, keep-alive arrays) for the C options, or (None, None) when all are off."""
    if dt_bias is None and not dt_softplus and dt_limit is None and not zoh:
        return None, None
    bias = None if dt_bias is None else _f32(dt_bias)
    assert bias is None or bias.shape == (H,)
    lo, hi = (0.0, 0.0) if dt_limit is None else (float(dt_limit[0]), float(dt_limit[1]))
    o = _Opts(_ptr(bias), int(bool(dt_softplus)), int(dt_limit is not None), lo, hi,
              int(bool(zoh)))
    return o, bias


def _load(path=None):
    """Load the oracle library (default: the built one; ``path`` loads another
    build of the same source, e.g. one compiled with a planted mistake)."""
    path = path or LIB_PATH
    if path not in _libs:
        if path == LIB_PATH and not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(path)
        fp, ip, dp = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p
        op = ctypes.POINTER(_Opts)
        lib.ssd_oracle_forward_ex.argtypes = [fp] * 7 + [ip] * 6 + [fp, ip, dp, dp, dp, ip, ip, op]
        lib.ssd_oracle_forward_ex.restype = ctypes.c_int
        lib.ssd_oracle_step_ex.argtypes = [dp] + [fp] * 6 + [ip] * 5 + [fp, ip, dp, ip, op]
        lib.ssd_oracle_step_ex.restype = ctypes.c_int
        lib.ssd_oracle_forward_varlen.argtypes = [fp] * 6 + [ip] * 5 + [fp, ip, fp, ip, dp, dp, ip, op]
        lib.ssd_oracle_forward_varlen.restype = ctypes.c_int
        lib.ssd_oracle_backward.argtypes = ([fp] * 6 + [dp, fp, dp] + [ip] * 6 + [fp, ip] +
                                            [dp] * 8 + [ip, op])
        lib.ssd_oracle_backward.restype = ctypes.c_int
        _libs[path] = lib
    return _libs[path]


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _f32(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data


def forward(x, dt, A, B, C, D=None, init=None, units=None, snap_every=0,
            want_state=True, nthreads=None, lib=None, dt_bias=None, dt_softplus=False,
            dt_limit=None, zoh=False):
    """Run the recurrence.

    Shapes: x [Bt,L,H,P], dt [Bt,L,H], B, C [Bt,L,G,N], A, D [H],
    init [Bt,H,P,N] (float64) or None. ``units`` lists flat b*H+h indices (default all).
    Returns (y [U,L,P], final state [U,P,N] or None, snapshots or None), float64.
    Snapshots hold the state after tokens snap_every-1, 2*snap_every-1, ...
    The dt options and ``zoh`` are described in the module docstring.
    """
    x, dt, A, B, C, D = map(_f32, (x, dt, A, B, C, D))
    init = None if init is None else np.ascontiguousarray(init, dtype=np.float64)
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (Bt, L, H) and B.shape == (Bt, L, G, N) and C.shape == B.shape
    assert A.shape == (H,) and (D is None or D.shape == (H,))
    assert init is None or init.shape == (Bt, H, P, N)
    if units is None:
        units_arr, U = None, Bt * H
    else:
        units_arr = np.ascontiguousarray(units, dtype=np.int32)
        U = units_arr.size
    y = np.empty((U, L, P), dtype=np.float64)
    st = np.empty((U, P, N), dtype=np.float64) if want_state else None
    nsnap = L // snap_every if snap_every > 0 else 0
    snaps = np.empty((U, nsnap, P, N), dtype=np.float64) if nsnap else None
    o, _keep = _opts(H, dt_bias, dt_softplus, dt_limit, zoh)
    rc = _load(lib).ssd_oracle_forward_ex(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init),
        Bt, L, H, P, G, N, _ptr(units_arr), U, _ptr(y), _ptr(st), _ptr(snaps),
        snap_every if nsnap else 0, nthreads or default_threads(),
        None if o is None else ctypes.byref(o))
    if rc != 0:
        raise RuntimeError(f"ssd_oracle_forward failed: {rc}")
    return y, st, snaps


def backward(x, dt, A, B, C, D, init, dy, dfinal=None, units=None, nthreads=None, lib=None,
             dt_bias=None, dt_softplus=False, dt_limit=None, zoh=False):
    """Gradients of loss = sum(dy * y) + sum(dfinal * final_state) for
    ``forward`` with the same inputs and options. Shapes as ``forward``; dy
    like x, dfinal like init (float64) or None.

    Returns a dict of float64 arrays shaped like the inputs, summed the way
    the inputs are shared: dx [Bt,L,H,P], ddt [Bt,L,H] (raw dt), dA [H],
    dB, dC [Bt,L,G,N] (summed over the heads of a group), dD [H],
    dinit [Bt,H,P,N], dbias [H]. With ``units`` (flat b*H + h) only those
    units are computed and the per-unit arrays are returned instead:
    dx [U,L,P], ddt [U,L], dA, dD, dbias [U], dB, dC [U,L,N], dinit [U,P,N].
    """
    x, dt, A, B, C, D, dy = map(_f32, (x, dt, A, B, C, D, dy))
    init = None if init is None else np.ascontiguousarray(init, dtype=np.float64)
    dfinal = None if dfinal is None else np.ascontiguousarray(dfinal, dtype=np.float64)
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dy.shape == x.shape and dt.shape == (Bt, L, H)
    if units is None:
        units_arr, U = None, Bt * H
    else:
        units_arr = np.ascontiguousarray(units, dtype=np.int32)
        U = units_arr.size
    out = {"dx": np.empty((U, L, P)), "ddt": np.empty((U, L)), "dA": np.empty(U),
           "dB": np.empty((U, L, N)), "dC": np.empty((U, L, N)), "dD": np.empty(U),
           "dinit": np.empty((U, P, N)), "dbias": np.empty(U)}
    o, _keep = _opts(H, dt_bias, dt_softplus, dt_limit, zoh)
    rc = _load(lib).ssd_oracle_backward(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init), _ptr(dy), _ptr(dfinal),
        Bt, L, H, P, G, N, _ptr(units_arr), U, *(out[k].ctypes.data for k in
        ("dx", "ddt", "dA", "dB", "dC", "dD", "dinit", "dbias")),
        nthreads or default_threads(), None if o is None else ctypes.byref(o))
    if rc != 0:
        raise RuntimeError(f"ssd_oracle_backward failed: {rc}")
    if units is not None:
        return out
    hpg = H // G
    return {
        "dx": out["dx"].reshape(Bt, H, L, P).transpose(0, 2, 1, 3),
        "ddt": out["ddt"].reshape(Bt, H, L).transpose(0, 2, 1),
        "dA": out["dA"].reshape(Bt, H).sum(axis=0),
        "dB": out["dB"].reshape(Bt, G, hpg, L, N).sum(axis=2).transpose(0, 2, 1, 3),
        "dC": out["dC"].reshape(Bt, G, hpg, L, N).sum(axis=2).transpose(0, 2, 1, 3),
        "dD": out["dD"].reshape(Bt, H).sum(axis=0),
        "dinit": out["dinit"].reshape(Bt, H, P, N),
        "dbias": out["dbias"].reshape(Bt, H).sum(axis=0),
    }


def forward_varlen(x, dt, A, B, C, D, cu_seqlens, units=None, nthreads=None, lib=None,
                   dt_bias=None, dt_softplus=False, dt_limit=None, zoh=False):
    """Packed sequences: x [1,L,H,P] (or [L,H,P]), dt [1,L,H], B, C [1,L,G,N];
    sequence k is tokens cu_seqlens[k] .. cu_seqlens[k+1]-1, each from the zero
    state. ``units`` lists heads (default all). Returns y [U,L,P] and the
    per-sequence final states [U,nseq,P,N], float64. Options as ``forward``.
    """
    x, dt, A, B, C, D = map(_f32, (x, dt, A, B, C, D))
    if x.ndim == 4:
        assert x.shape[0] == 1, "packed sequences use batch 1"
        x, dt, B, C = x[0], dt[0], B[0], C[0]
    L, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    assert dt.shape == (L, H) and B.shape == (L, G, N) and C.shape == B.shape
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    nseq = cu.size - 1
    if units is None:
        units_arr, U = None, H
    else:
        units_arr = np.ascontiguousarray(units, dtype=np.int32)
        U = units_arr.size
    y = np.empty((U, L, P), dtype=np.float64)
    st = np.empty((U, nseq, P, N), dtype=np.float64)
    o, _keep = _opts(H, dt_bias, dt_softplus, dt_limit, zoh)
    rc = _load(lib).ssd_oracle_forward_varlen(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), L, H, P, G, N, _ptr(cu), nseq,
        _ptr(units_arr), U, _ptr(y), _ptr(st), nthreads or default_threads(),
        None if o is None else ctypes.byref(o))
    if rc != 0:
        raise RuntimeError(f"ssd_oracle_forward_varlen failed: {rc}")
    return y, st


def step(state, x, dt, A, B, C, D=None, units=None, nthreads=None, lib=None,
         dt_bias=None, dt_softplus=False, dt_limit=None, zoh=False):
    """One recurrent step. ``state`` [U,P,N] float64 is updated in place.

    x [Bt,H,P], dt [Bt,H], B, C [Bt,G,N]. Returns y [U,P] float64.
    The dt options and ``zoh`` are those of ``forward``.
    """
    x, dt, A, B, C, D = map(_f32, (x, dt, A, B, C, D))
    Bt, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    assert state.dtype == np.float64 and state.flags.c_contiguous
    if units is None:
        units_arr, U = None, Bt * H
    else:
        units_arr = np.ascontiguousarray(units, dtype=np.int32)
        U = units_arr.size
    assert state.shape == (U, P, N)
    y = np.empty((U, P), dtype=np.float64)
    o, _keep = _opts(H, dt_bias, dt_softplus, dt_limit, zoh)
    rc = _load(lib).ssd_oracle_step_ex(
        _ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
        Bt, H, P, G, N, _ptr(units_arr), U, _ptr(y), nthreads or default_threads(),
        None if o is None else ctypes.byref(o))
    if rc != 0:
        raise RuntimeError(f"ssd_oracle_step failed: {rc}")
    return y


def quadratic(x, dt, A, B, C, D=None, init=None, weights=None):
    """Dual quadratic form, O(L^2) per (batch, head); small inputs only.

    ``weights`` [Bt,L,H] replaces dt as the weight of the input term below
    (the decay still uses dt); None means the weights are dt.

    For each (b, h) with group g = h // (H // G):
      a_k  = dt_k A_h,  cs_i = sum_{k<=i} a_k
      L_ij = exp(cs_i - cs_j) for j <= i else 0      (= exp(sum_{k=j+1..i} a_k))
      y    = (L o (C_g B_g^T)) (dt o x) + D x + exp(cs_i) C_i . h0
      h_L  = exp(cs_{L-1}) h0 + sum_j exp(cs_{L-1} - cs_j) dt_j x_j B_j^T
    Returns y [Bt,L,H,P] and the final state [Bt,H,P,N], float64.
    """
    x = np.asarray(x, np.float64)
    dt = np.asarray(dt, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    wt = dt if weights is None else np.asarray(weights, np.float64)
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.zeros((Bt, L, H, P))
    hf = np.zeros((Bt, H, P, N))
    idx = np.arange(L)
    causal = idx[:, None] >= idx[None, :]
    for b in range(Bt):
        for h in range(H):
            g = h // (H // G)
            cs = np.cumsum(dt[b, :, h] * A[h])
            Lmat = np.where(causal, np.exp(np.where(causal, cs[:, None] - cs[None, :], 0.0)), 0.0)
            M = Lmat * (C[b, :, g, :] @ B[b, :, g, :].T)
            u = wt[b, :, h, None] * x[b, :, h, :]
            y[b, :, h, :] = M @ u
            w = np.exp(cs[-1] - cs) * wt[b, :, h]
            hf[b, h] = (x[b, :, h, :] * w[:, None]).T @ B[b, :, g, :]
            if D is not None:
                y[b, :, h, :] += float(D[h]) * x[b, :, h, :]
            if init is not None:
                h0 = np.asarray(init[b, h], np.float64)
                y[b, :, h, :] += np.exp(cs)[:, None] * (C[b, :, g, :] @ h0.T)
                hf[b, h] += np.exp(cs[-1]) * h0
    return y, hf


def chunk_cumsum(dt, A, chunk):
    """Within-chunk inclusive prefix sums of dt*A, float64.

    dt [Bt,L,H], A [H] -> s [Bt,H,L] with s_t = sum_{k=cQ..t} dt_k A_h for t in
    chunk c = t // Q; the last chunk may be short.
    """
    dt = np.asarray(dt, np.float64)
    a = np.transpose(dt * np.asarray(A, np.float64)[None, None, :], (0, 2, 1))
    Bt, H, L = a.shape
    s = np.empty_like(a)
    for c0 in range(0, L, chunk):
        s[:, :, c0:c0 + chunk] = np.cumsum(a[:, :, c0:c0 + chunk], axis=2)
    return s
