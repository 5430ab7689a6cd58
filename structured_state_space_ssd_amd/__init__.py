"""MI355X-native Mamba-2 SSD layer: chunked forward pass and recurrent decode.

Thin Python front end over libssd.so (include/ssd.h). Tensors are torch tensors
on the GPU; work is enqueued on torch's current stream. Nothing here computes:
the functions check tensor metadata, allocate outputs / workspace with torch,
and call the C ABI.
"""
from __future__ import annotations

import ctypes

import torch

from . import _native
from ._native import SSDError, check, dtype_code, ptr, stream_handle

__all__ = ["forward", "forward_plan", "plan_info", "backward", "forward_varlen", "step", "options", "workspace_size", "chunk_cumsum", "chunk_state",
           "state_passing", "chunk_cb", "chunk_scan", "SSDError", "stages"]

HEADDIM = 64


def _req(t, name, dtype=None, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _opt(t, name, dtype=torch.float32):
    return None if t is None else _req(t, name, dtype)


def options(dt_bias=None, dt_softplus=False, dt_limit=None, zoh=False):
    """ssd_options for the C ABI, or None when every option is off.

    dt_bias: GPU float32 [H] added to dt first; dt_softplus: apply
    log(1 + e^dt) next; dt_limit = (lo, hi): clamp last; zoh: weight the
    input term by (exp(dt A) - 1) / A instead of dt. The returned structure
    points at dt_bias's memory and holds a reference to the tensor, so the
    memory stays allocated as long as the structure is alive.
    """
    if dt_bias is None and not dt_softplus and dt_limit is None and not zoh:
        return None
    if dt_bias is not None:
        _req(dt_bias, "dt_bias", torch.float32)
    lo, hi = (0.0, 0.0) if dt_limit is None else (float(dt_limit[0]), float(dt_limit[1]))
    o = _native.SsdOptions(None if dt_bias is None else dt_bias.data_ptr(), int(bool(dt_softplus)),
                           int(dt_limit is not None), lo, hi,
                           _native.SSD_DISC_ZOH if zoh else _native.SSD_DISC_EULER)
    o.bias_tensor = dt_bias  # keeps the bias memory alive with the structure
    return o


def _optref(o):
    return None if o is None else ctypes.byref(o)


def workspace_size(batch, seqlen, nheads, headdim, ngroups, dstate, chunk, dtype=torch.bfloat16) -> int:
    return int(_native.lib.ssd_forward_workspace_size(batch, seqlen, nheads, headdim, ngroups, dstate,
                                                      chunk, dtype_code(dtype)))


def plan_info(batch, seqlen, nheads, headdim, ngroups, dstate, chunk, dtype=torch.bfloat16,
              dt=None) -> dict:
    """How ``forward`` runs for these sizes (ssd_forward_plan_info): path
    ("single_pass" or "stages"), segments S, pieces K, block_tokens,
    segment_blocks, piece_blocks and workspace_bytes. ``dt`` (a tensor, or
    None for an aligned pointer) matters only through its alignment."""
    p = _native.SsdPlan()
    addr = dt.data_ptr() if dt is not None else 256
    rc = int(_native.lib.ssd_forward_plan_info(batch, seqlen, nheads, headdim, ngroups, dstate,
                                               chunk, dtype_code(dtype), addr, ctypes.byref(p)))
    check(rc, "ssd_forward_plan_info")
    return {"path": "single_pass" if p.path == 1 else "stages", "segments": p.segments,
            "pieces": p.pieces, "block_tokens": p.block_tokens,
            "segment_blocks": p.segment_blocks, "piece_blocks": p.piece_blocks,
            "kernel_dstate": p.kernel_dstate, "workspace_bytes": int(p.workspace_bytes)}


def forward_plan(batch, seqlen, nheads, headdim, ngroups, dstate, chunk, dtype=torch.bfloat16,
                 dt=None) -> int:
    """Segments per sequence of the single-pass forward for these sizes (0: the
    stage kernels run; ssd_forward_plan). ``dt`` (a tensor, or None for an
    aligned pointer) matters only through its alignment."""
    ptr = dt.data_ptr() if dt is not None else 256
    r = int(_native.lib.ssd_forward_plan(batch, seqlen, nheads, headdim, ngroups, dstate, chunk,
                                         dtype_code(dtype), ptr))
    if r < 0:
        _native.check(r, "ssd_forward_plan")
    return r


def _shape(t, name, want):
    """ValueError unless tensor t (None allowed) has shape ``want``."""
    if t is not None and tuple(t.shape) != tuple(want):
        raise ValueError(f"{name} must have shape {tuple(want)}, got {tuple(t.shape)}")


def _params(A, D, H, dt_bias=None):
    """A and D (nullable) float32 [H], dt_bias (nullable) float32 [H]."""
    _shape(A, "A", (H,))
    _shape(D, "D", (H,))
    _shape(dt_bias, "dt_bias", (H,))


def forward(x, dt, A, B, C, D=None, chunk=256, init_state=None, return_final_state=False,
            workspace=None, y=None, events=None, dt_bias=None, dt_softplus=False,
            dt_limit=None, zoh=False):
    """y = SSD(x, dt, A, B, C, D) over whole sequences.

    x [Bt,L,H,P], dt [Bt,L,H], B, C [Bt,L,G,N] (all float32 or all bfloat16),
    A, D [H] float32, init_state [Bt,H,P,N] float32 or None.
    dt_bias, dt_softplus, dt_limit, zoh: see ``options``.
    Returns y (and the final state [Bt,H,P,N] float32 if requested).
    ``events``: optional sequence of 6 torch.cuda.Event(enable_timing=True) or None;
    the library records them around its five stages (see ssd_forward_timed),
    skipping the None entries.
    """
    # shapes first (the C ABI takes sizes, not shapes: a mis-shaped tensor
    # would be read or written out of bounds), then device, layout and dtype
    for t, n in ((x, "x"), (dt, "dt"), (A, "A"), (B, "B"), (C, "C")):
        if t is None:
            raise ValueError(f"{n} is required")
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [Bt, L, H, P] and B [Bt, L, G, N]")
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if tuple(dt.shape) != (Bt, L, H) or tuple(B.shape) != (Bt, L, G, N) or C.shape != B.shape:
        raise ValueError("shape mismatch among x, dt, B, C")
    _params(A, D, H, dt_bias)
    _shape(init_state, "init_state", (Bt, H, P, N))
    _shape(y, "y", x.shape)
    _req(x, "x")
    dt_ = dtype_code(x.dtype)
    _req(dt, "dt", x.dtype)
    _req(B, "B", x.dtype)
    _req(C, "C", x.dtype)
    _req(A, "A", torch.float32)
    _opt(D, "D")
    _opt(init_state, "init_state")
    if y is None:
        y = torch.empty_like(x)
    _req(y, "y", x.dtype)
    fs = torch.empty((Bt, H, P, N), dtype=torch.float32, device=x.device) if return_final_state else None
    need = plan_info(Bt, L, H, P, G, N, chunk, x.dtype, dt)["workspace_bytes"]
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    ev = _event_array(events, 6)
    opts = options(dt_bias, dt_softplus, dt_limit, zoh)
    rc = _native.lib.ssd_forward_ex(
        ptr(x), ptr(dt), ptr(A), ptr(B), ptr(C), ptr(D), Bt, L, H, P, G, N, chunk, dt_,
        ptr(init_state), ptr(y), ptr(fs), ptr(workspace), workspace.numel() * workspace.element_size(), _optref(opts),
        stream_handle(x.device), ev)
    check(rc, "ssd_forward")
    return (y, fs) if return_final_state else y


def _event_array(events, n):
    """ctypes array of n hipEvent_t from torch.cuda.Event (or None) entries."""
    if events is None:
        return None
    if len(events) != n:
        raise ValueError(f"events must hold {n} entries (torch.cuda.Event or None)")
    for e in events:
        if e is not None and not e.cuda_event:
            e.record()  # torch creates the HIP event on its first record
    return (ctypes.c_void_p * n)(*[e.cuda_event if e is not None else None for e in events])


def backward(x, dt, A, B, C, D, dy, init_state=None, dfinal_state=None, dt_bias=None,
             dt_softplus=False, dt_limit=None, zoh=False, workspace=None, want_dinit=True,
             events=None):
    """Gradients of sum(dy * y) + sum(dfinal_state * final_state) for
    ``forward`` with the same inputs and options (ssd_backward).
    ``events``: optional sequence of 5 torch.cuda.Event or None, recorded
    around the backward's phases (see ssd_backward_timed).

    Returns a dict: dx, ddt, dB, dC (input dtype, shaped like x, dt, B, C),
    dA, dD (float32 [H]), dinit (float32 [Bt,H,P,N], or None if not
    want_dinit) and, when dt_bias is given, ddt_bias (float32 [H]).
    """
    for t, n in ((x, "x"), (dt, "dt"), (A, "A"), (B, "B"), (C, "C"), (dy, "dy")):
        if t is None:
            raise ValueError(f"{n} is required")
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [Bt, L, H, P] and B [Bt, L, G, N]")
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if (tuple(dt.shape) != (Bt, L, H) or tuple(B.shape) != (Bt, L, G, N) or C.shape != B.shape
            or dy.shape != x.shape):
        raise ValueError("shape mismatch among x, dt, B, C, dy")
    _params(A, D, H, dt_bias)
    _shape(init_state, "init_state", (Bt, H, P, N))
    _shape(dfinal_state, "dfinal_state", (Bt, H, P, N))
    _req(x, "x")
    dt_ = dtype_code(x.dtype)
    for t, n in ((dt, "dt"), (B, "B"), (C, "C"), (dy, "dy")):
        _req(t, n, x.dtype)
    _req(A, "A", torch.float32)
    _opt(D, "D")
    _opt(init_state, "init_state")
    _opt(dfinal_state, "dfinal_state")
    dev = x.device
    out = {"dx": torch.empty_like(x), "ddt": torch.empty_like(dt), "dB": torch.empty_like(B),
           "dC": torch.empty_like(C), "dA": torch.empty(H, dtype=torch.float32, device=dev),
           "dD": torch.empty(H, dtype=torch.float32, device=dev),
           "dinit": (torch.empty((Bt, H, P, N), dtype=torch.float32, device=dev)
                     if want_dinit else None)}
    if dt_bias is not None:
        out["ddt_bias"] = torch.empty(H, dtype=torch.float32, device=dev)
    need = int(_native.lib.ssd_backward_workspace_size(Bt, L, H, P, G, N, dt_))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    opts = options(dt_bias, dt_softplus, dt_limit, zoh)
    rc = _native.lib.ssd_backward_timed(
        ptr(x), ptr(dt), ptr(A), ptr(B), ptr(C), ptr(D), ptr(init_state), ptr(dy),
        ptr(dfinal_state), Bt, L, H, P, G, N, dt_, ptr(out["dx"]), ptr(out["ddt"]),
        ptr(out["dA"]), ptr(out["dB"]), ptr(out["dC"]), ptr(out["dD"]), ptr(out["dinit"]),
        ptr(out.get("ddt_bias")), ptr(workspace), workspace.numel() * workspace.element_size(),
        _optref(opts), stream_handle(dev), _event_array(events, 5))
    check(rc, "ssd_backward")
    return out


def forward_varlen(x, dt, A, B, C, D, cu_seqlens, chunk=256, return_seq_states=False,
                   workspace=None, y=None, dt_bias=None, dt_softplus=False, dt_limit=None,
                   zoh=False):
    """Packed variable-length sequences: x [L,H,P] or [1,L,H,P], dt [L,H] or
    [1,L,H], B, C [L,G,N] or [1,L,G,N]; sequence k is tokens
    cu_seqlens[k] .. cu_seqlens[k+1]-1 (GPU int32 [nseq+1], starting at 0,
    non-decreasing, ending at L), each from the zero state.
    Returns y (shaped like x) and, if requested, the per-sequence final states
    [nseq,H,P,N] float32. Options as ``forward``.
    """
    for t, n in ((x, "x"), (dt, "dt"), (A, "A"), (B, "B"), (C, "C"), (cu_seqlens, "cu_seqlens")):
        if t is None:
            raise ValueError(f"{n} is required")
    squeeze = x.dim() == 3
    xs = x.unsqueeze(0) if squeeze else x
    if xs.dim() != 4 or xs.shape[0] != 1:
        raise ValueError("packed sequences use batch 1: x [L, H, P] or [1, L, H, P]")
    _, L, H, P = xs.shape
    if B.dim() not in (3, 4) or (B.dim() == 4 and B.shape[0] != 1):
        raise ValueError("B must be [L, G, N] or [1, L, G, N]")
    G, N = B.shape[-2], B.shape[-1]
    if (dt.numel() != L * H or B.numel() != L * G * N or C.shape != B.shape
            or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2):
        raise ValueError("shape mismatch among x, dt, B, C, cu_seqlens")
    _params(A, D, H, dt_bias)
    _shape(y, "y", x.shape)
    _req(x, "x")
    dt_ = dtype_code(x.dtype)
    _req(dt, "dt", x.dtype)
    _req(B, "B", x.dtype)
    _req(C, "C", x.dtype)
    _req(A, "A", torch.float32)
    _opt(D, "D")
    _req(cu_seqlens, "cu_seqlens", torch.int32)
    nseq = cu_seqlens.numel() - 1
    if y is None:
        y = torch.empty_like(x)
    ss = (torch.empty((nseq, H, P, N), dtype=torch.float32, device=x.device)
          if return_seq_states else None)
    need = int(_native.lib.ssd_forward_varlen_workspace_size(L, H, P, G, N, chunk, dt_))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    opts = options(dt_bias, dt_softplus, dt_limit, zoh)
    rc = _native.lib.ssd_forward_varlen(
        ptr(x), ptr(dt), ptr(A), ptr(B), ptr(C), ptr(D), ptr(cu_seqlens), nseq, L, H, P, G, N,
        chunk, dt_, ptr(y), ptr(ss), ptr(workspace), workspace.numel() * workspace.element_size(), _optref(opts),
        stream_handle(x.device))
    check(rc, "ssd_forward_varlen")
    return (y, ss) if return_seq_states else y


def step(state, x, dt, A, B, C, D=None, y=None, dt_bias=None, dt_softplus=False, dt_limit=None,
         zoh=False):
    """One decode step; updates state [Bt,H,P,N] float32 in place, returns y [Bt,H,P].

    x [Bt,H,P], dt [Bt,H], B, C [Bt,G,N] (float32 or bfloat16), A, D [H] float32.
    dt_bias, dt_softplus, dt_limit, zoh: see ``options``.
    """
    for t, n in ((state, "state"), (x, "x"), (dt, "dt"), (A, "A"), (B, "B"), (C, "C")):
        if t is None:
            raise ValueError(f"{n} is required")
    if x.dim() != 3 or B.dim() != 3:
        raise ValueError("x must be [Bt, H, P] and B [Bt, G, N]")
    Bt, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    if (tuple(state.shape) != (Bt, H, P, N) or tuple(dt.shape) != (Bt, H)
            or tuple(B.shape) != (Bt, G, N) or C.shape != B.shape):
        raise ValueError("shape mismatch among state, x, dt, B, C")
    _params(A, D, H, dt_bias)
    _shape(y, "y", x.shape)
    _req(state, "state", torch.float32)
    _req(x, "x")
    dt_ = dtype_code(x.dtype)
    _req(dt, "dt", x.dtype)
    _req(B, "B", x.dtype)
    _req(C, "C", x.dtype)
    _req(A, "A", torch.float32)
    _opt(D, "D")
    if y is None:
        y = torch.empty_like(x)
    _req(y, "y", x.dtype)
    opts = options(dt_bias, dt_softplus, dt_limit, zoh)
    rc = _native.lib.ssd_step_ex(ptr(state), ptr(x), ptr(dt), ptr(A), ptr(B), ptr(C), ptr(D),
                                 Bt, H, P, G, N, dt_, ptr(y), _optref(opts),
                                 stream_handle(x.device))
    check(rc, "ssd_step")
    return y


# ---- stage-by-stage entry points (what forward enqueues) --------------------

def _nc(L, Q):
    return (L + Q - 1) // Q


def chunk_cumsum(dt, A, chunk, out=None, delta=None, return_delta=False, opts=None):
    """dA_cumsum [Bt,H,nC*Q] float32: within-chunk prefix sums of dt*A (dt
    after the preprocessing in ``opts``, an ``options(...)`` result or None);
    with return_delta (or a given ``delta`` buffer), also each token's input
    weight as float32 in the same layout (zero past the end)."""
    _req(dt, "dt")
    Bt, L, H = dt.shape
    shape = (Bt, H, _nc(L, chunk) * chunk)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=dt.device)
    if delta is None and return_delta:
        delta = torch.empty(shape, dtype=torch.float32, device=dt.device)
    rc = _native.lib.ssd_chunk_cumsum(ptr(dt), ptr(_req(A, "A", torch.float32)), Bt, L, H, chunk,
                                      dtype_code(dt.dtype), ptr(out),
                                      ptr(_opt(delta, "delta")), _optref(opts),
                                      stream_handle(dt.device))
    check(rc, "ssd_chunk_cumsum")
    return (out, delta) if delta is not None else out


def chunk_state(x, B, delta, dA_cumsum, chunk, out=None):
    """states [Bt,nC,H,P,N] float32: each chunk's contribution from a zero state
    (delta: chunk_cumsum's input weights)."""
    Bt, L, H, P = _req(x, "x").shape
    G, N = B.shape[2], B.shape[3]
    if out is None:
        out = torch.empty((Bt, _nc(L, chunk), H, P, N), dtype=torch.float32, device=x.device)
    rc = _native.lib.ssd_chunk_state(ptr(x), ptr(_req(B, "B", x.dtype)),
                                     ptr(_req(delta, "delta", torch.float32)),
                                     ptr(_req(dA_cumsum, "dA_cumsum", torch.float32)), Bt, L, H, P, G,
                                     N, chunk, dtype_code(x.dtype), ptr(out), stream_handle(x.device))
    check(rc, "ssd_chunk_state")
    return out


def state_passing(states, dA_cumsum, seqlen, chunk, init_state=None, out=None, final_state=None,
                  dtype=torch.float32):
    """chunk_init [Bt,nC,H,P,N] (state entering each chunk) in ``dtype`` (the
    forward's input dtype: bf16 or float32); optional float32 final state."""
    Bt, nC, H, P, N = _req(states, "states", torch.float32).shape
    if out is None:
        out = torch.empty(states.shape, dtype=dtype, device=states.device)
    rc = _native.lib.ssd_state_passing(ptr(states), ptr(_req(dA_cumsum, "dA_cumsum", torch.float32)),
                                       ptr(_opt(init_state, "init_state")), Bt, seqlen, H, P, N, chunk,
                                       dtype_code(out.dtype), ptr(out),
                                       ptr(_opt(final_state, "final_state")),
                                       stream_handle(states.device))
    check(rc, "ssd_state_passing")
    return out


def chunk_cb(B, C, chunk, out=None):
    """C B^T tiles of every chunk (opaque layout, read by chunk_scan)."""
    Bt, L, G, N = _req(B, "B").shape
    n = int(_native.lib.ssd_chunk_cb_size(Bt, L, G, chunk, dtype_code(B.dtype)))
    if out is None:
        out = torch.empty(max(n, 1), dtype=torch.uint8, device=B.device)
    rc = _native.lib.ssd_chunk_cb(ptr(B), ptr(_req(C, "C", B.dtype)), Bt, L, G, N, chunk,
                                  dtype_code(B.dtype), ptr(out), stream_handle(B.device))
    check(rc, "ssd_chunk_cb")
    return out


def chunk_scan(x, delta, dA_cumsum, B, C, cb, D, chunk_init, chunk, y=None):
    """y [Bt,L,H,P]: intra-chunk product + state-to-output + D x
    (delta: chunk_cumsum's input weights).

    bfloat16 forms C B^T on chip from B (cb may be None); float32 reads the
    C B^T tiles of chunk_cb (B may be None)."""
    Bt, L, H, P = _req(x, "x").shape
    G, N = C.shape[2], C.shape[3]
    if y is None:
        y = torch.empty_like(x)
    bf16 = x.dtype == torch.bfloat16
    rc = _native.lib.ssd_chunk_scan(ptr(x), ptr(_req(delta, "delta", torch.float32)),
                                    ptr(_req(dA_cumsum, "dA_cumsum", torch.float32)),
                                    ptr(_req(B, "B", x.dtype) if bf16 else B),
                                    ptr(_req(C, "C", x.dtype)), ptr(cb if bf16 else _req(cb, "cb")),
                                    ptr(_opt(D, "D")), ptr(_req(chunk_init, "chunk_init", x.dtype)),
                                    Bt, L, H, P, G, N, chunk, dtype_code(x.dtype), ptr(y),
                                    stream_handle(x.device))
    check(rc, "ssd_chunk_scan")
    return y


def stages(x, dt, A, B, C, D=None, chunk=256, init_state=None, dt_bias=None, dt_softplus=False,
           dt_limit=None, zoh=False):
    """Run the forward stages one call at a time; returns a dict with every
    intermediate (dA_cumsum, delta, states, chunk_init, final_state, cb) and y."""
    Bt, L, H, P = x.shape
    N = B.shape[3]
    opts = options(dt_bias, dt_softplus, dt_limit, zoh)
    s, delta = chunk_cumsum(dt, A, chunk, return_delta=True, opts=opts)
    st = chunk_state(x, B, delta, s, chunk)
    fs = torch.empty((Bt, H, P, N), dtype=torch.float32, device=x.device)
    ci = state_passing(st, s, L, chunk, init_state=init_state, final_state=fs, dtype=x.dtype)
    cb = chunk_cb(B, C, chunk)
    y = chunk_scan(x, delta, s, B, C, cb, D, ci, chunk)
    return {"dA_cumsum": s, "delta": delta, "states": st, "chunk_init": ci, "final_state": fs,
            "cb": cb, "y": y}
