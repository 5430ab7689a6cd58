"""SSD layer benchmark on one MI355X.

One step = one full SSD forward over the Mamba-2 2.7B-shaped layer: batch 8,
L 2048, 80 heads x P 64, N 64, one B/C group, chunk argument 256, bf16
inputs, fp32 accumulation, inputs resident in HBM. Prints ONE JSON line.

The timed region is cold: before each step, outside its events, a 1 GiB
buffer is read, so neither L2 nor the 256 MB Infinity Cache holds any input;
HIP events around each forward (and between its kernels) on the launch
stream give its time, and ``value`` is tokens over the mean. The warm figure
(back-to-back forwards, inputs partly from the Infinity Cache) is reported
beside it as ``forward_warm``.

For this shape the library runs the whole forward as its single-pass kernel
(forward_onepass, 64-token blocks whatever the chunk argument); with few
(batch, head) pairs it adds a segment-state kernel first (segment_states);
shapes outside the single-pass kernel run the stages chunk_cumsum,
chunk_state, state_passing, chunk_cb, chunk_scan. The library's own plan
(ssd_forward_plan_info) says which, and the bench line's config reports it.

Also reported: the tiny, large-state and long-sequence forwards (cold, per
kernel), the stage kernels called one by one at the 2.7B and large-state
shapes (state passing's HBM GB/s among them), the forward with every
step-size option, packed variable-length sequences, the backward (with the
chunk-gradient kernel's roofline), the decode step (256 x 80 heads, P 64,
N 128, fp32 state, 64 consecutive tokens) and a plain device copy's
bandwidth. Roofline figures use algorithmic bytes / flops (what the method
must read, write and compute), not executed ones. The CPU baseline is the
fp64 oracle (test infrastructure) on the same workload, timed on this host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--no-cpu]
       python bench.py --trace-run | --counters [--backward] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSD layer fwd tokens/s + MFMA util (2.7B-shape, L=2048); decode step GB/s"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (no sparsity)
FP32_PEAK_TFLOPS = 157.3    # MI355X fp32 matrix
STAGES = ["chunk_cumsum", "chunk_state", "state_passing", "chunk_cb", "chunk_scan"]
ONEPASS = ["forward_onepass"]
ONEPASS_SEG = ["segment_states", "forward_onepass"]  # sequences cut into segments
SOURCE_OF = {"forward_onepass": "fwd_onepass", "segment_states": "fwd_onepass"}  # -> csrc/ file
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


# ---------------------------------------------------------------- accounting

def plan_of(w, dt=None):
    """The library's own plan for this forward (ssd_forward_plan_info): path,
    segments S, pieces K, block length, blocks per segment, workspace bytes."""
    import torch
    import structured_state_space_ssd_amd as ssd
    return ssd.plan_info(w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate, w.chunk,
                         torch.bfloat16 if w.dtype == "bf16" else torch.float32, dt)


def stages_of(w):
    """Kernels the forward launches, in order (the library's plan decides)."""
    p = plan_of(w)
    if p["path"] == "stages":
        return STAGES
    return ONEPASS if p["segments"] == 1 else ONEPASS_SEG


def onepass_accounting(w):
    """Algorithmic bytes and flops of the single-pass forward kernel (and, when
    the sequences are cut into S segments, of the segment-state kernel).

    Bytes: x and dt read, y written (bf16), B and C read once per group, A and
    D (float32) once per head; nothing else leaves the chip. Flops (multiply +
    add = 2) of the chunked algorithm at the kernel's 64-token blocks:
    (T+1)P per token-head for the causal block products, 2NP for the state to
    output, 2NP for the state update, 2P for the D term, and (T+1)N per token
    per group for the causal C B^T products. With S segments the segment-state
    kernel reads x, dt and B over the first S-1 segments and writes their
    pieces' states (float32 P x N and a log2-decay per (batch, head, piece),
    2NP flops per token-head), which the single-pass kernel reads back."""
    Bt, L, H, P, G, N = w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate
    p = plan_of(w)
    T = p["block_tokens"]
    S, k, per_seg = p["segments"], max(1, p["pieces"]), p["segment_blocks"]
    tok = Bt * L
    seg_states = p["workspace_bytes"]  # exactly the pieces' states and decays
    nbytes = 2 * tok * H * P * 2 + tok * H * 2 + 2 * tok * G * N * 2 + 2 * H * 4 + seg_states
    flops = tok * H * ((T + 1) * P + 4 * N * P + 2 * P) + tok * G * (T + 1) * N
    acc = {"forward_onepass": {"bytes": nbytes, "flops": flops}}
    if S > 1:
        pre = Bt * (S - 1) * per_seg * T  # tokens of the first S-1 segments
        acc["segment_states"] = {"bytes": pre * H * (P * 2 + 2) + pre * G * N * 2 + H * 4 +
                                          seg_states,
                                 "flops": pre * H * 2 * N * P}
    return acc


def stage_accounting(w, fused=None):
    """Algorithmic bytes and flops per launch of each forward stage.

    Bytes: every input read once and every output written once, at its storage
    width (bf16 2 B for x, dt, B, C, y and, in bf16 runs, chunk_init; float32
    4 B for A, D, dA_cumsum, the per-token input weights delta and the chunk
    states). B and C are counted once per group, not per head. Stages 2 and 4
    read delta (written by stage 1, the size of dA_cumsum) in place of dt.
    The C B^T tiles (float path: chunk_cb output, chunk_scan input) are
    counted once each way; the bf16 chunk scan forms them on chip (from B and
    C, counted once per group) and chunk_cb is not launched. Flops (multiply +
    add = 2): chunk_state 2PN per token-head;
    chunk_scan (Q+1)P (causal masked product: Q(Q+1)/2 pairs x 2P per
    chunk-head) + 2NP (state to output) + 2P (skip) per token-head; chunk_cb
    (Q+1)N per token per group (causal C B^T); state_passing 2PN per
    chunk-head element pair. ``fused``: whether stages 2 and 3 run as one
    kernel (None: the forward's own rule, bf16 with batch * nheads >= 512;
    the stage entry points called one by one never fuse).
    """
    Bt, L, H, P, G, N, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate, w.chunk
    e = 2 if w.dtype == "bf16" else 4
    nC = -(-L // Q)
    tok = Bt * L
    x = tok * H * P * e
    dt = tok * H * e
    bc = tok * G * N * e
    s = Bt * H * nC * Q * 4
    st = Bt * nC * H * P * N * 4
    ci = Bt * nC * H * P * N * e  # chunk_init, stored in the operand type
    send = Bt * H * nC * 4
    nt = Q // 16
    cb = Bt * nC * G * (nt // 2) * (nt // 2 + 1) * 512 * e  # causal C B^T tiles
    cb_flops = tok * G * (Q + 1) * N
    scan_flops = tok * H * ((Q + 1) * P + 2 * N * P + 2 * P)
    if w.dtype == "bf16":
        # the bf16 chunk scan forms C B^T on chip from B and C: no chunk_cb launch
        cb_stage = {"bytes": 0, "flops": 0}
        scan = {"bytes": x + x + 2 * s + 2 * bc + ci + H * 4, "flops": scan_flops + cb_flops}
    else:
        cb_stage = {"bytes": 2 * bc + cb, "flops": cb_flops}
        scan = {"bytes": x + x + 2 * s + bc + cb + ci + H * 4, "flops": scan_flops}
    # stage 1 writes dA_cumsum and the float32 input weights (delta), same size
    cumsum = {"bytes": dt + H * 4 + 2 * s, "flops": tok * H * 2}
    state = {"bytes": x + bc + 2 * s + st, "flops": tok * H * 2 * P * N}
    passing = {"bytes": st + ci + send, "flops": Bt * nC * H * P * N * 2}
    if fused is None:
        fused = w.dtype == "bf16" and Bt * H >= 512
    if fused:
        # one kernel for stages 2 and 3: reads x, B, s and delta, writes
        # chunk_init and the final state; no per-chunk states
        fin = Bt * H * P * N * 4
        state = {"bytes": x + bc + 2 * s + ci + fin,
                 "flops": state["flops"] + passing["flops"]}
        passing = {"bytes": 0, "flops": 0}
    return {"chunk_cumsum": cumsum, "chunk_state": state, "state_passing": passing,
            "chunk_cb": cb_stage, "chunk_scan": scan}


def accounting(w):
    """Per-kernel algorithmic bytes and flops of the forward as the library runs it."""
    return onepass_accounting(w) if plan_of(w)["path"] == "single_pass" else stage_accounting(w)


def backward_accounting(w):
    """Algorithmic bytes and flops of the backward's chunk-gradient kernel (one
    launch). Bytes: it reads x and dy (input dtype), B and C once per group,
    the prefix sums s and weights w (float32 per token-head, chunk-padded),
    the state entering each chunk H_c and the adjoint leaving it G_{c+1}
    (operand type, [Bt][nC][H][P][N]); it writes dx (input dtype), ds and dw
    (float32 per token-head), the dB and dC partial sums (float32 per head
    block) and dD per chunk-head. Flops (multiply + add = 2) per token-head:
    the causal dy.x^T blocks and dx (2 (Q+1) P), the causal dB and dC
    products (2 (Q+1) N), the state terms G B, G^T x, H^T dy, H C (8 N P);
    plus (Q+1) N per token and group for the causal C.B^T blocks. Q is the
    backward's own chunk length (128 for N <= 64, else 64)."""
    Bt, L, H, P, G, N = w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate
    e = 2 if w.dtype == "bf16" else 4
    Q = 128 if N <= 64 else 64
    nC = -(-L // Q)
    nU = Bt * nC * G
    nblk = max(1, min(H // G, -(-256 // nU)))
    tok = Bt * L
    tokh = Bt * H * nC * Q * 4
    states = Bt * nC * H * P * N * e
    nbytes = (3 * tok * H * P * e + 2 * tok * G * N * e + 2 * tokh + 2 * states + 2 * tokh +
              2 * nblk * tok * G * N * 4 + Bt * nC * H * 4)
    flops = tok * H * (2 * (Q + 1) * P + 2 * (Q + 1) * N + 8 * N * P) + tok * G * (Q + 1) * N
    return {"chunk_bwd": {"bytes": nbytes, "flops": flops, "chunk": Q, "head_blocks": nblk}}


def decode_accounting(w):
    Bt, H, P, G, N = w.batch, w.nheads, w.headdim, w.ngroups, w.dstate
    e = 2 if w.dtype == "bf16" else 4
    state = Bt * H * P * N * 4
    inputs = Bt * H * P * e + Bt * H * e + 2 * Bt * G * N * e + 2 * H * 4
    return {"bytes": 2 * state + inputs + Bt * H * P * e, "flops": Bt * H * P * N * 5}


def kernel_source_digest(name):
    """Digest of a kernel's source file and the shared header, comments and
    whitespace left out (a counter record stays valid across comment edits,
    not across code changes)."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "structured_state_space_ssd_amd", "csrc")
    for f in (f"{SOURCE_OF.get(name, name)}.hip", "ssd_common.h"):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload="mamba2_2.7b"):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current source of the kernel; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(workload, {}).get(kernel)
    if not rec or rec.get("source_digest") != kernel_source_digest(kernel):
        return None
    return rec.get("bytes_per_launch")


def kernel_figures(a, seconds, dtype):
    """Per-kernel figures from algorithmic bytes / flops and a time."""
    gbs = a["bytes"] / seconds / 1e9
    tfl = a["flops"] / seconds / 1e12
    peak_f = BF16_PEAK_TFLOPS if dtype == "bf16" else FP32_PEAK_TFLOPS
    intensity = a["flops"] / a["bytes"] if a["bytes"] else 0.0
    applicable = min(peak_f, intensity * HBM_PEAK_GBS / 1e3)  # TFLOP/s roof at this intensity
    return {"us": round(seconds * 1e6, 2), "alg_bytes": a["bytes"], "alg_flops": a["flops"],
            "GB_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "TFLOP_s": round(tfl, 2), "mfma_frac": round(tfl / peak_f, 4),
            "roofline_frac": round(tfl / applicable, 4) if applicable else None}


# ---------------------------------------------------------------- GPU timing

_GEN = {}


def gen(w):
    """W.generate(w), drawn once per workload and run (a shallow copy: callers
    may replace entries)."""
    import ssd_workloads as W
    if w.name not in _GEN:
        _GEN[w.name] = W.generate(w)
    return dict(_GEN[w.name])


def upload(d):
    import numpy as np
    import torch
    import ssd_workloads as W
    out = {}
    for k, t in d.items():
        if t is None:
            out[k] = None
        elif isinstance(t, W.Tensor):
            if t.dtype == "bf16":
                out[k] = torch.from_numpy(t.dev.view(np.int16)).view(torch.bfloat16).cuda()
            else:
                out[k] = torch.from_numpy(t.dev).cuda()
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(t)).cuda()
    return out


def spin_up(call, seconds=0.15):
    """Back-to-back calls for about `seconds`, untimed: the GPU raises its
    clocks only under sustained load (the first tens of milliseconds run up to
    20% slower), so every timed region starts with the clocks up."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            call()
        torch.cuda.synchronize()


class Flush:
    """Reads a 1 GiB buffer (a sum: clean lines only, so the next kernel does
    not also write back a flush's dirty lines), which leaves neither L2 nor
    the 256 MB Infinity Cache holding any input of the next kernel."""

    def __init__(self, nbytes=1 << 30):
        import torch
        self.buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        self.sink = torch.zeros((), dtype=torch.float32, device="cuda")

    def __call__(self):
        self.sink += self.buf.sum()


COLD = ("cold caches: before each step, outside its events, a 1 GiB buffer is read, so "
        "that neither L2 nor the 256 MB Infinity Cache holds any input")


def _stats(v):
    v = sorted(v)
    n = len(v)
    return {"mean": sum(v) / n, "median": v[n // 2], "p10": v[n // 10], "p90": v[(9 * n) // 10]}


def time_forward_cold(w, steps, warmup, flush=None):
    """The timed region: ``warmup`` untimed cold forwards, then ``steps`` cold
    forwards between two synchronizations. Before each, outside its events, a
    1 GiB read (Flush); around each forward and between its kernels, HIP
    events on the launch stream (ssd_forward_timed). Returns the forward's
    mean / median / p10 / p90 (ms), each kernel's mean (ms) and the host wall
    time of the region (flushes included)."""
    import torch
    import ssd_workloads as W
    import structured_state_space_ssd_amd as ssd

    g = upload(gen(w))
    x, dt, A, B, C, D = (g[k] for k in ("x", "dt", "A", "B", "C", "D"))
    need = plan_of(w, dt)["workspace_bytes"]
    ws = torch.empty(max(1, need), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    flush = flush or Flush()
    stages = stages_of(w)
    ns = len(stages)
    mk = lambda: torch.cuda.Event(enable_timing=True)
    pad = lambda evs: list(evs) + [None] * (len(STAGES) + 1 - len(evs))
    call = lambda ev=None: ssd.forward(x, dt, A, B, C, D, chunk=w.chunk, workspace=ws, y=y,
                                       events=ev)
    spin_up(call)
    for _ in range(warmup):
        flush()
        call()
    evs = [[mk() for _ in range(ns + 1)] for _ in range(steps)]
    for e in evs:
        for ev in e:
            ev.record()  # create the HIP events before the timed region
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        flush()
        call(pad(e))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd = _stats([e[0].elapsed_time(e[ns]) for e in evs])
    per = {stages[i]: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / steps for i in range(ns)}
    del x, dt, B, C, y, ws, g
    return {"forward_ms": fwd, "kernel_ms": per, "wall_ms": wall * 1e3 / steps}


def time_forward_warm(w, steps, warmup):
    """Back-to-back forwards over the same resident inputs (host clock around
    ``steps`` of them, after ``warmup``): part of the inputs then comes from
    the Infinity Cache when they fit in it."""
    import torch
    import ssd_workloads as W
    import structured_state_space_ssd_amd as ssd

    g = upload(gen(w))
    x, dt, A, B, C, D = (g[k] for k in ("x", "dt", "A", "B", "C", "D"))
    ws = torch.empty(max(1, plan_of(w, dt)["workspace_bytes"]), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    call = lambda: ssd.forward(x, dt, A, B, C, D, chunk=w.chunk, workspace=ws, y=y)
    spin_up(call)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def time_stages_cold(w, reps=20, flush=None):
    """The forward's stage kernels called one by one through their entry
    points (ssd_chunk_cumsum, ssd_chunk_state, ssd_state_passing,
    ssd_chunk_cb for float32, ssd_chunk_scan: the chunked form with the
    per-chunk states in HBM, never fused), cold (Flush before each pass),
    with HIP events between them. Returns each stage's mean time (ms)."""
    import torch
    import ssd_workloads as W
    import structured_state_space_ssd_amd as ssd

    g = upload(gen(w))
    x, dt, A, B, C, D = (g[k] for k in ("x", "dt", "A", "B", "C", "D"))
    Bt, L, H, P, N, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.chunk
    nC = -(-L // Q)
    f32 = torch.float32
    s = torch.empty((Bt, H, nC * Q), dtype=f32, device="cuda")
    delta = torch.empty_like(s)
    st = torch.empty((Bt, nC, H, P, N), dtype=f32, device="cuda")
    ci = torch.empty((Bt, nC, H, P, N), dtype=x.dtype, device="cuda")
    fs = torch.empty((Bt, H, P, N), dtype=f32, device="cuda")
    y = torch.empty_like(x)
    bf16 = w.dtype == "bf16"
    cb = None if bf16 else ssd.chunk_cb(B, C, Q)

    def run(ev):
        ev[0].record()
        ssd.chunk_cumsum(dt, A, Q, out=s, delta=delta)
        ev[1].record()
        ssd.chunk_state(x, B, delta, s, Q, out=st)
        ev[2].record()
        ssd.state_passing(st, s, L, Q, out=ci, final_state=fs, dtype=x.dtype)
        ev[3].record()
        if not bf16:
            ssd.chunk_cb(B, C, Q, out=cb)
        ev[4].record()
        ssd.chunk_scan(x, delta, s, B, C, cb, D, ci, Q, y=y)
        ev[5].record()

    flush = flush or Flush()
    mk = lambda: torch.cuda.Event(enable_timing=True)
    spin_up(lambda: run([mk() for _ in range(6)]), 0.1)
    evs = [[mk() for _ in range(6)] for _ in range(reps)]
    for e in evs:
        flush()
        run(e)
    torch.cuda.synchronize()
    out = {}
    for i, name in enumerate(STAGES):
        if name == "chunk_cb" and bf16:
            continue
        out[name] = sum(e[i].elapsed_time(e[i + 1]) for e in evs) / reps
    out["_total"] = sum(e[0].elapsed_time(e[5]) for e in evs) / reps
    return out


def time_forward_options(w, steps, warmup):
    """Whole-forward time (host clock, no events, after spin_up) with every
    step-size option on: per-head bias, softplus, clamp to [4e-3, 3e-2] and the zero-order-hold
    input weight, on the same shapes (raw dt from generate_dt_raw)."""
    import torch
    import ssd_workloads as W
    import structured_state_space_ssd_amd as ssd

    d = gen(w)
    r = W.generate_dt_raw(w)
    d["dt"], d["dt_bias"] = r["dt"], r["dt_bias"]
    g = upload(d)
    x = g["x"]
    ws = torch.empty(max(1, plan_of(w, g["dt"])["workspace_bytes"]), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty_like(x)
    kw = dict(chunk=w.chunk, workspace=ws, y=y, dt_bias=g["dt_bias"], dt_softplus=True,
              dt_limit=(4e-3, 3e-2), zoh=True)
    args = [g[k] for k in ("x", "dt", "A", "B", "C", "D")]
    spin_up(lambda: ssd.forward(*args, **kw))
    for _ in range(warmup):
        ssd.forward(*args, **kw)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        ssd.forward(*args, **kw)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def varlen_workload():
    """The 2.7B layer's tokens (8 x 2048) packed into one row of sequences of
    1 .. 4096 tokens (ssd_workloads.packed_cu_seqlens)."""
    import ssd_workloads as W
    w = W.Workload("packed_2.7b", 1, 16384, 80, 64, 1, 64, 256, "bf16", 1 / 8, 1e-3, 1e-1,
                   seed=860)
    return w, W.packed_cu_seqlens(w.seqlen, 4096, seed=861)


def time_forward_varlen(steps, warmup):
    """Whole-forward time (host clock) of the packed variable-length forward,
    per-sequence final states included."""
    import torch
    import ssd_workloads as W
    import structured_state_space_ssd_amd as ssd

    w, cu = varlen_workload()
    g = upload(gen(w))
    cu_g = torch.from_numpy(cu).cuda()
    x = g["x"]
    ws = torch.empty(int(ssd._native.lib.ssd_forward_varlen_workspace_size(
        w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate, w.chunk, 1)), dtype=torch.uint8,
        device="cuda")
    y = torch.empty_like(x)
    args = [g[k] for k in ("x", "dt", "A", "B", "C", "D")] + [cu_g]
    kw = dict(chunk=w.chunk, workspace=ws, y=y, return_seq_states=True)
    spin_up(lambda: ssd.forward_varlen(*args, **kw))
    for _ in range(warmup):
        ssd.forward_varlen(*args, **kw)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        ssd.forward_varlen(*args, **kw)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    return w, cu, ms


BWD_PHASES = ["recompute", "adjoint", "chunk_bwd", "reductions"]


def time_backward(w, steps, warmup, cold=False, flush=None):
    """Whole-backward time: gradients of every input for the workload's
    forward, with a final-state gradient and every dt option off. Warm: host
    clock over back-to-back backwards. Cold (Flush before each, outside the
    events): the mean of HIP events around each backward and its phases
    (ssd_backward_timed)."""
    import torch
    import ssd_workloads as W
    import structured_state_space_ssd_amd as ssd

    d = gen(w)
    d.update(W.generate_grads(w))
    g = upload(d)
    ws = torch.empty(int(ssd._native.lib.ssd_backward_workspace_size(
        w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate, 1 if w.dtype == "bf16" else 0)),
        dtype=torch.uint8, device="cuda")
    args = [g[k] for k in ("x", "dt", "A", "B", "C", "D", "dy")]
    kw = dict(init_state=g["init"], dfinal_state=g["dfinal"], workspace=ws)
    spin_up(lambda: ssd.backward(*args, **kw))
    for _ in range(warmup):
        ssd.backward(*args, **kw)
    torch.cuda.synchronize()
    if not cold:
        t0 = time.perf_counter()
        for _ in range(steps):
            ssd.backward(*args, **kw)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps
    flush = flush or Flush()
    mk = lambda: torch.cuda.Event(enable_timing=True)
    evs = [[mk() for _ in range(5)] for _ in range(steps)]
    for e in evs:
        flush()
        ssd.backward(*args, events=e, **kw)
    torch.cuda.synchronize()
    out = {name: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / steps
           for i, name in enumerate(BWD_PHASES)}
    out["_total"] = sum(e[0].elapsed_time(e[4]) for e in evs) / steps
    return out


def time_decode(w, warmup=3):
    import torch
    import ssd_workloads as W
    import structured_state_space_ssd_amd as ssd

    d = W.generate(w)
    g = upload(d)
    state = g["init"]
    x, dt, A, B, C, D = (g[k] for k in ("x", "dt", "A", "B", "C", "D"))
    y = torch.empty_like(x[0])
    for t in range(warmup):
        ssd.step(state, x[t], dt[t], A, B[t], C[t], D, y=y)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(w.seqlen + 1)]
    ev[0].record()
    for t in range(w.seqlen):
        ssd.step(state, x[t], dt[t], A, B[t], C[t], D, y=y)
        ev[t + 1].record()
    torch.cuda.synchronize()
    per = [ev[t].elapsed_time(ev[t + 1]) for t in range(w.seqlen)]
    return {"mean_ms": sum(per) / len(per), "min_ms": min(per), "max_ms": max(per)}


def hbm_probe(nbytes=1 << 30, reps=5):
    """A plain 1 GiB device-to-device copy (torch), larger than the 256 MB
    Infinity Cache, timed with events: the bandwidth a simple streaming kernel
    reaches on this machine, reported beside the 8 TB/s peak as context."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return {"copy_bytes": nbytes, "us": round(ms * 1e3, 1),
            "read_plus_write_GB_s": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


def cpu_baseline(w, min_seconds=1.5):
    """The fp64 oracle (as it stands) on the same workload, on this host.

    A bounded sample: whole forward passes over the workload, repeated until
    at least ``min_seconds`` of wall time (about 10-30 s of CPU work on the
    threads it uses)."""
    import oracle
    d = gen(w)
    n = oracle.default_threads()
    passes, sec = 0, 0.0
    while passes == 0 or sec < min_seconds:
        t0 = time.perf_counter()
        oracle.forward(d["x"].val, d["dt"].val, d["A"], d["B"].val, d["C"].val, d["D"], None,
                       want_state=True, nthreads=n)
        sec += time.perf_counter() - t0
        passes += 1
    return {"value": round(passes * w.tokens / sec, 1), "unit": "tokens/s", "cores": n,
            "kind": "oracle",
            "sample": f"{passes} pass(es) of the whole {w.name} forward (batch {w.batch} x L "
                      f"{w.seqlen}, all {w.batch * w.nheads} (batch, head) units, y and final "
                      f"state), fp64 recurrence on {n} threads, {sec:.2f} s wall"}


def counters_run(w, backward=False):
    """A short, fixed sequence of launches for counter collection: a plain
    1 GiB device copy (it calibrates the byte counters), a few cold forwards
    of the workload (and with ``backward`` a few cold backwards), and the
    decode steps."""
    import torch
    copy_bytes = 1 << 30
    src = torch.empty(copy_bytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(2):
        dst.copy_(src)  # reads and writes exactly copy_bytes each
    torch.cuda.synchronize()
    print(f"[counters] copy of {copy_bytes} bytes x2 done", file=sys.stderr, flush=True)
    del src, dst
    time_forward_cold(w, steps=3, warmup=1)
    print("[counters] forward x4 done", file=sys.stderr, flush=True)
    if backward:
        time_backward(w, steps=2, warmup=0, cold=True)
        print("[counters] backward done", file=sys.stderr, flush=True)
    else:
        time_decode(W_decode(), warmup=0)
        print("[counters] decode done", file=sys.stderr, flush=True)


def trace_run(w, steps, warmup):
    """Only the headline's timed region (warmup + cold timed forwards, each
    after its 1 GiB read), for a kernel trace whose last ``steps`` dispatches
    of each forward kernel are exactly the timed ones."""
    r = time_forward_cold(w, steps, warmup)
    print(json.dumps({"workload": w.name, "steps": steps, "warmup": warmup,
                      "forward_us_mean": round(r["forward_ms"]["mean"] * 1e3, 2),
                      "kernel_us": {k: round(v * 1e3, 2) for k, v in r["kernel_ms"].items()}}),
          flush=True)


# ---------------------------------------------------------------- profile summaries
#
# The rocprofv3 runs these read (OUT is any scratch directory; WL a workload
# name: mamba2_2.7b, large_state, long_seq):
TRACE_CMD = ('rocprofv3 --kernel-trace --stats --output-format csv -d "$OUT/trace_$WL" -o trace '
             '-- python bench.py --trace-run --workload $WL --steps 50 --warmup 10 '
             '> "$OUT/trace_$WL.log"')
FETCH_CMD = ('rocprofv3 --pmc FETCH_SIZE --output-format csv -d "$OUT/fetch_$WL" -o fetch '
             '-- python bench.py --counters --workload $WL')
WRITE_CMD = ('rocprofv3 --pmc WRITE_SIZE --output-format csv -d "$OUT/write_$WL" -o write '
             '-- python bench.py --counters --workload $WL')
UTIL_CMDS = ('rocprofv3 --pmc MfmaUtil VALUBusy LdsUtil --output-format csv -d "$OUT/util_$WL" '
             '-o util -- python bench.py --counters --workload $WL',
             'rocprofv3 --pmc MfmaFlopsBF16 --output-format csv -d "$OUT/mops_$WL" -o mops '
             '-- python bench.py --counters --workload $WL')
# kernel-name fragment -> kernel, first match wins (the fused stage-2+3 kernel
# fills the chunk_state interval of the forward)
KERNEL_OF = {"segment_states_kernel": "segment_states", "segment_chain_kernel": "segment_chain",
             "ssd_forward_onepass": "forward_onepass", "onepass_varlen_prep": "packed: token int4s",
             "chunk_cumsum_kernel": "chunk_cumsum", "chunk_state_passing": "chunk_state",
             "state_passing_kernel": "state_passing", "chunk_state": "chunk_state",
             "chunk_cb_kernel": "chunk_cb", "chunk_scan": "chunk_scan",
             "decode_step_kernel": "decode_step", "chunk_bwd_kernel": "chunk_bwd",
             "bwd_dt_kernel": "backward: dt, A, bias", "bwd_reduce_kernel": "backward: dB, dC sums",
             "bwd_head_sum_kernel": "backward: per-head sums", "varlen_seg": "packed: token masks"}
CALIBRATION_KERNEL = "__amd_rocclr_copyBuffer"  # the 1 GiB device copy of --counters
COPY_BYTES = 1 << 30


def _stage_of(kernel_name):
    for k, v in KERNEL_OF.items():
        if k in kernel_name:
            return v
    return None


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(names)


def summarize_trace(trace_csv, run_log):
    """Markdown table of a --kernel-trace run of ``bench.py --trace-run``: for
    each kernel, its dispatch count and the average, min and max duration of
    its last ``steps`` dispatches (exactly the timed cold forwards), beside the
    run's own event timings."""
    rows = _read_csv(trace_csv)
    run = None
    with open(run_log) as f:
        for line in f:
            if line.startswith("{"):
                run = json.loads(line)
    steps = run["steps"]
    per = {}
    for r in rows:
        name = _col(r, "Kernel_Name", "Name")
        t = (int(_col(r, "End_Timestamp", "End")) - int(_col(r, "Start_Timestamp", "Start"))) / 1e3
        per.setdefault(name, []).append((int(_col(r, "Start_Timestamp", "Start")), t))
    wl = run["workload"]
    out = [f"# Kernel trace: the timed cold forwards of `{wl}`", "",
           f"`bench.py --trace-run` runs {run['warmup']} untimed and {steps} timed forwards, each",
           "after a 1 GiB read that leaves no input in L2 or the Infinity Cache (the bench",
           "line's timed region), and nothing else on the GPU but the reads' own reduction",
           "kernels. Durations are from the per-dispatch kernel trace: the last "
           f"{steps} dispatches of each kernel are the timed ones.", "",
           "Commands, from the repository root on one MI355X:", "", "```",
           "cd /tmp && export TMPDIR=/tmp && cd -", f"WL={wl}", TRACE_CMD,
           f'python bench.py --summarize-trace "$OUT/trace_$WL/trace_kernel_trace.csv" '
           f'"$OUT/trace_$WL.log"', "```", "",
           "| kernel | role | dispatches | avg us (timed) | min us | max us | bench event avg us |",
           "|---|---|---|---|---|---|---|"]
    for name, v in sorted(per.items(), key=lambda kv: -sum(t for _, t in kv[1])):
        role = _stage_of(name)
        if role is None:
            continue
        v.sort()
        last = [t for _, t in v[-steps:]]
        ev = run["kernel_us"].get(role, "")
        short = name.split("(")[0].replace("void ", "")
        out.append(f"| `{short}` | {role} | {len(v)} | {sum(last) / len(last):.2f} | "
                   f"{min(last):.2f} | {max(last):.2f} | {ev} |")
    out += ["", f"The run's own figure: {run['forward_us_mean']} us per cold forward (HIP events "
                f"around each), kernels {json.dumps(run['kernel_us'])}."]
    return "\n".join(out)


def _summary_accounting(workload):
    import ssd_workloads as W
    w = W.WORKLOADS[workload]
    acc = dict(accounting(w))
    acc.update({k: v for k, v in backward_accounting(w).items()})
    acc["decode_step"] = decode_accounting(W_decode())
    return acc


def summarize_traffic(fetch_csv, write_csv, workload="mamba2_2.7b"):
    """HBM bytes per launch of each kernel from FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch), each scaled by what the same counter reads for the
    plain 1 GiB device copy of the same run. Returns (markdown, json dict)."""
    per = {}
    for tag, path in (("fetch", fetch_csv), ("write", write_csv)):
        for r in _read_csv(path):
            name = r["Kernel_Name"]
            key = CALIBRATION_KERNEL if name == CALIBRATION_KERNEL else _stage_of(name)
            if key is None:
                continue
            per.setdefault(key, {}).setdefault(tag, []).append(float(r["Counter_Value"]))
    cal = per[CALIBRATION_KERNEL]
    f_scale = COPY_BYTES / 1024 / max(cal["fetch"])
    w_scale = COPY_BYTES / 1024 / max(cal["write"])
    acc = _summary_accounting(workload)
    rec = {"_calibration": {"kernel": CALIBRATION_KERNEL, "copy_bytes": COPY_BYTES,
                            "fetch_kib": max(cal["fetch"]), "write_kib": max(cal["write"]),
                            "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
                            "commands": [FETCH_CMD, WRITE_CMD]}}
    out = [f"# HBM traffic per launch: SSD kernels (`{workload}`)",
           "", "Commands, from the repository root on one MI355X (add `--backward` to both",
           "counter runs for the backward's kernels):", "", "```",
           "cd /tmp && export TMPDIR=/tmp && cd -", f"WL={workload}",
           f"timeout -s KILL 60 {FETCH_CMD}", f"timeout -s KILL 60 {WRITE_CMD}",
           'python bench.py --summarize-traffic "$OUT/fetch_$WL/fetch_counter_collection.csv" '
           f'"$OUT/write_$WL/write_counter_collection.csv" --workload $WL', "```", "",
           f"Calibration: the 1 GiB device copy reads FETCH_SIZE {max(cal['fetch']):.0f} KiB and "
           f"WRITE_SIZE {max(cal['write']):.0f} KiB, so FETCH_SIZE is scaled by {f_scale:.3f} and "
           f"WRITE_SIZE by {w_scale:.3f}.", "",
           "| kernel | dispatches | fetch MB | write MB | HBM MB / launch | algorithmic MB | ratio |",
           "|---|---|---|---|---|---|---|"]
    for k in ONEPASS_SEG + STAGES + ["chunk_bwd", "decode_step"]:
        if k not in acc:
            continue
        if k not in per or "fetch" not in per[k] or "write" not in per[k]:
            continue
        fk = sum(per[k]["fetch"]) / len(per[k]["fetch"])
        wk = sum(per[k]["write"]) / len(per[k]["write"])
        b = fk * 1024 * f_scale + wk * 1024 * w_scale
        alg = acc[k]["bytes"]
        rec[k] = {"fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                  "bytes_per_launch": round(b), "alg_bytes": alg,
                  "source_digest": kernel_source_digest(k)}
        out.append(f"| {k} | {len(per[k]['fetch'])} | {fk * 1024 * f_scale / 1e6:.1f} | "
                   f"{wk * 1024 * w_scale / 1e6:.1f} | {b / 1e6:.1f} | {alg / 1e6:.1f} | {b / alg:.2f} |")
    return "\n".join(out), rec


def summarize_util(util_csv, mops_csv, workload="mamba2_2.7b"):
    """Markdown table of the MFMA-busy, VALU-busy and LDS counters (percent of
    the kernel's active cycles, averaged over its dispatches) and the executed
    bf16 MFMA flops against the algorithmic ones, per kernel."""
    per = {}
    for path in (util_csv, mops_csv):
        for r in _read_csv(path):
            k = _stage_of(r["Kernel_Name"])
            if k is None:
                continue
            per.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    acc = _summary_accounting(workload)
    out = [f"# MFMA, VALU and LDS utilisation: SSD kernels (`{workload}`)", "",
           "rocprofv3 derived counters, each the average over the kernel's dispatches:",
           "MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs), VALUBusy and",
           "LdsUtil likewise in percent of busy cycles; MfmaFlopsBF16 = 512 x",
           "SQ_INSTS_VALU_MFMA_MOPS_BF16, the executed bf16 MFMA flops per launch, beside",
           "the algorithmic flops the accounting counts (the executed ones include the",
           "zero-padded halves of causal tiles and the D x products).", "",
           "Commands, from the repository root on one MI355X (add `--backward` to both",
           "counter runs for the backward's kernels):", "", "```",
           "cd /tmp && export TMPDIR=/tmp && cd -", f"WL={workload}"] + \
          [f"timeout -s KILL 60 {c}" for c in UTIL_CMDS] + \
          ['python bench.py --summarize-util "$OUT/util_$WL/util_counter_collection.csv" '
           f'"$OUT/mops_$WL/mops_counter_collection.csv" --workload $WL', "```", "",
           "| kernel | dispatches | MfmaUtil % | VALUBusy % | LdsUtil % | executed MFMA GFLOP "
           "| algorithmic GFLOP |", "|---|---|---|---|---|---|---|"]
    avg = lambda v: sum(v) / len(v) if v else float("nan")
    for k in ONEPASS_SEG + STAGES + ["chunk_bwd"]:
        if k not in per or k not in acc:
            continue
        c = per[k]
        out.append(f"| {k} | {len(c.get('MfmaUtil', []))} | {avg(c.get('MfmaUtil', [])):.1f} | "
                   f"{avg(c.get('VALUBusy', [])):.1f} | {avg(c.get('LdsUtil', [])):.1f} | "
                   f"{avg(c.get('MfmaFlopsBF16', [])) / 1e9:.2f} | {acc[k]['flops'] / 1e9:.2f} |")
    return "\n".join(out)


def W_decode():
    import ssd_workloads as W
    return W.WORKLOADS["decode"]


def _workload_line(w, r, acc):
    """Figures of one cold-timed forward workload."""
    kern = {k: kernel_figures(acc[k], v * 1e-3, w.dtype) for k, v in r["kernel_ms"].items()
            if acc[k]["bytes"]}
    f = r["forward_ms"]
    p = plan_of(w)
    return {"us_per_forward": round(f["mean"] * 1e3, 2), "p10_us": round(f["p10"] * 1e3, 2),
            "p90_us": round(f["p90"] * 1e3, 2),
            "tokens_per_s": round(w.tokens / (f["mean"] * 1e-3), 1),
            "plan": {k: p[k] for k in ("path", "segments", "pieces", "block_tokens")},
            "kernels": kern}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="mamba2_2.7b")
    ap.add_argument("--quick", action="store_true",
                    help="the headline only: skip the other workloads and the stage kernels")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--forward-only", action="store_true",
                    help="only the cold and warm forward of --workload (no JSON contract line)")
    ap.add_argument("--counters", action="store_true",
                    help="short run for rocprofv3 counter collection: a plain 1 GiB device copy "
                         "that calibrates the byte counters, a few forwards of --workload, and the "
                         "decode steps (with --backward: a few backwards instead)")
    ap.add_argument("--backward", action="store_true", help="with --counters: the backward")
    ap.add_argument("--trace-run", action="store_true",
                    help="only the timed region of --workload (for a kernel trace)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_CSV", "RUN_LOG"),
                    help="print the markdown summary of a rocprofv3 --kernel-trace run of --trace-run")
    ap.add_argument("--summarize-util", nargs=2, metavar=("UTIL_CSV", "MOPS_CSV"),
                    help="print the MFMA / VALU / LDS utilisation summary of two rocprofv3 "
                         "--pmc runs")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM-traffic summary of two rocprofv3 --pmc runs and record "
                         "it in profiles/hbm_traffic.json")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(*args.summarize_trace))
        return
    if args.summarize_util:
        print(summarize_util(*args.summarize_util, workload=args.workload))
        return
    if args.summarize_traffic:
        md, rec = summarize_traffic(*args.summarize_traffic, workload=args.workload)
        try:
            with open(TRAFFIC_FILE) as f:
                allrec = json.load(f)
        except (OSError, ValueError):
            allrec = {}
        allrec.setdefault(args.workload, {}).update(rec)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(allrec, f, indent=1)
            f.write("\n")
        print(md)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this SSD build has no multi-GPU path "
              "(batch/head sharding needs no communication; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import ssd_workloads as W
    import structured_state_space_ssd_amd  # noqa: F401  (fails loudly if libssd.so is missing)

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    w = W.WORKLOADS[args.workload]
    if args.counters:
        counters_run(w, args.backward)
        return
    if args.trace_run:
        trace_run(w, args.steps, args.warmup)
        return
    say = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)
    say(f"{w.name}: {args.warmup} warmup + {args.steps} timed cold forwards")
    flush = Flush()
    cold = time_forward_cold(w, args.steps, args.warmup, flush)
    f = cold["forward_ms"]
    ms = f["mean"]
    acc = accounting(w)
    kernels = {k: kernel_figures(acc[k], v * 1e-3, w.dtype) for k, v in cold["kernel_ms"].items()
               if acc[k]["bytes"]}
    dom = max(kernels, key=lambda k: kernels[k]["us"])
    dom_s = cold["kernel_ms"][dom] * 1e-3
    dom_gbs = acc[dom]["bytes"] / dom_s / 1e9
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                "us_per_launch": round(dom_s * 1e6, 2), "alg_bytes_per_launch": acc[dom]["bytes"],
                "traffic": measured_traffic(dom, w.name), "cache": "cold"}
    say(f"cold forward {ms * 1e3:.1f} us (median {f['median'] * 1e3:.1f}); " +
        ", ".join(f"{k} {v['us']:.1f} us" for k, v in kernels.items()))

    if args.forward_only:
        print(json.dumps({"workload": w.name, "cold_us": round(ms * 1e3, 2),
                          "kernels": {k: {"us": v["us"], "hbm_frac": v["hbm_frac"]}
                                      for k, v in kernels.items()},
                          "warm_us": round(time_forward_warm(w, args.steps, 3) * 1e3, 2),
                          "plan": plan_of(w)}), flush=True)
        return
    warm_ms = time_forward_warm(w, args.steps, max(3, args.warmup // 4))
    warm = {"protocol": "back-to-back forwards over the same resident inputs, host clock around "
                        f"{args.steps} of them; inputs that fit in the 256 MB Infinity Cache are "
                        "partly read from it",
            "us_per_forward": round(warm_ms * 1e3, 2),
            "tokens_per_s": round(w.tokens / (warm_ms * 1e-3), 1),
            "hbm_frac": round(sum(a["bytes"] for a in acc.values()) / (warm_ms * 1e-3) / 1e9 /
                              HBM_PEAK_GBS, 4)}
    say(f"warm forward {warm_ms * 1e3:.1f} us")

    extra, stage_lines = {}, {}
    if not args.quick:
        for name in ("tiny_f32", "large_state", "long_seq"):
            wl = W.WORKLOADS[name]
            r = time_forward_cold(wl, 20, 5, flush)
            extra[name] = _workload_line(wl, r, accounting(wl))
            say(f"{name}: {extra[name]['us_per_forward']} us cold; " +
                ", ".join(f"{k} {v['us']:.1f} us ({v['hbm_frac']:.3f} of HBM)"
                          for k, v in extra[name]["kernels"].items()))
        for name in ("mamba2_2.7b", "large_state"):
            wl = W.WORKLOADS[name]
            r = time_stages_cold(wl, 20, flush)
            sa = stage_accounting(wl, fused=False)
            stage_lines[name] = {
                "protocol": "the stage entry points one by one (per-chunk states in HBM, never "
                            "fused), cold, HIP events between them, mean of 20",
                "us_total": round(r.pop("_total") * 1e3, 2),
                "kernels": {k: kernel_figures(sa[k], v * 1e-3, wl.dtype) for k, v in r.items()}}
            say(f"{name} stage kernels: " + ", ".join(
                f"{k} {v['us']:.1f} us ({v['hbm_frac']:.3f} of HBM, {v['mfma_frac']:.3f} of MFMA)"
                for k, v in stage_lines[name]["kernels"].items()))

    opt_ms = time_forward_options(w, max(10, args.steps // 2), 3)
    options = {"options": "dt_bias + softplus + clamp + zero-order hold (warm, back to back)",
               "us_per_forward": round(opt_ms * 1e3, 2),
               "tokens_per_s": round(w.tokens / (opt_ms * 1e-3), 1)}
    say(f"forward with every step-size option: {opt_ms * 1e3:.1f} us")

    wv, cu, vl_ms = time_forward_varlen(max(10, args.steps // 2), 3)
    varlen = {"workload": f"{wv.seqlen} tokens (the 2.7B layer's 8 x 2048) packed as {cu.size - 1} "
                          "sequences of 1 .. 4096 tokens, bf16, per-sequence final states "
                          "(warm, back to back)",
              "us_per_forward": round(vl_ms * 1e3, 2),
              "tokens_per_s": round(wv.seqlen / (vl_ms * 1e-3), 1)}
    say(f"packed variable-length forward: {vl_ms * 1e3:.1f} us")

    bw_ms = time_backward(w, max(10, args.steps // 2), 3)
    bwc = time_backward(w, 20, 3, cold=True, flush=flush)
    ba = backward_accounting(w)
    cb = kernel_figures(ba["chunk_bwd"], bwc["chunk_bwd"] * 1e-3, w.dtype)
    cb.update({"chunk": ba["chunk_bwd"]["chunk"], "head_blocks": ba["chunk_bwd"]["head_blocks"]})
    backward = {"workload": "gradients of x, dt, A, B, C, D and the initial state, same shapes",
                "us_per_backward": round(bw_ms * 1e3, 2),
                "tokens_per_s": round(w.tokens / (bw_ms * 1e-3), 1),
                "cold_us_per_backward": round(bwc["_total"] * 1e3, 2),
                "cold_phase_us": {k: round(bwc[k] * 1e3, 2) for k in BWD_PHASES},
                "chunk_bwd": cb}
    say(f"backward: {bw_ms * 1e3:.1f} us warm, {bwc['_total'] * 1e3:.1f} us cold; chunk_bwd "
        f"{cb['us']} us ({cb['hbm_frac']:.3f} of HBM)")

    wd = W.WORKLOADS["decode"]
    dec = time_decode(wd)
    da = decode_accounting(wd)
    dec_gbs = da["bytes"] / (dec["mean_ms"] * 1e-3) / 1e9
    decode = {"workload": "decode: batch 256, 80 heads x P 64, N 128, fp32 state, bf16 inputs, 64 steps",
              "us_per_step": round(dec["mean_ms"] * 1e3, 2), "GB_s": round(dec_gbs, 1),
              "hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4), "alg_bytes_per_step": da["bytes"],
              "tokens_per_s": round(wd.batch / (dec["mean_ms"] * 1e-3))}
    say(f"decode {decode['us_per_step']} us/step, {decode['GB_s']} GB/s")

    del flush
    probe = hbm_probe()
    say(f"1 GiB device copy: {probe['read_plus_write_GB_s']} GB/s (read + write)")

    cpu = None
    if not args.no_cpu:
        say("cpu baseline (fp64 oracle)...")
        cpu = cpu_baseline(w)

    p = plan_of(w)
    out = {
        "metric": METRIC,
        "value": round(w.tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; shapes and distributions of the named workload)",
        "config": {"workload": "SSD layer forward, Mamba-2 2.7B shape", "batch": w.batch,
                   "seq_len": w.seqlen, "nheads": w.nheads, "headdim": w.headdim,
                   "dstate": w.dstate, "ngroups": w.ngroups, "chunk": w.chunk,
                   "path": p["path"], "block_tokens": p["block_tokens"],
                   "segments": p["segments"], "cache": "cold", "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "timing": {"protocol": COLD + "; HIP events around each forward and between its "
                               "kernels on the launch stream; value = tokens / mean",
                   "median_us": round(f["median"] * 1e3, 2), "p10_us": round(f["p10"] * 1e3, 2),
                   "p90_us": round(f["p90"] * 1e3, 2),
                   "wall_ms_per_step_with_flush": round(cold["wall_ms"], 4)},
        "kernels": kernels,
        "forward_warm": warm,
        "forward_with_options": options,
        "forward_varlen": varlen,
        "backward": backward,
        "decode": decode,
        "hbm_copy_probe": probe,
    }
    if extra:
        out["other_workloads"] = extra
    if stage_lines:
        out["stage_kernels"] = stage_lines
        out["state_passing"] = {k: {"GB_s": v["kernels"]["state_passing"]["GB_s"],
                                    "hbm_frac": v["kernels"]["state_passing"]["hbm_frac"],
                                    "us": v["kernels"]["state_passing"]["us"]}
                                for k, v in stage_lines.items()}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
