"""SSD layer benchmark on one MI355X.

One step = one full SSD forward over the Mamba-2 2.7B-shaped layer: batch 8,
L 2048, 80 heads x P 64, N 64, one B/C group, chunk 256, bf16 inputs, fp32
accumulation, inputs already resident in HBM. Prints ONE JSON line. For this
shape the library runs the whole forward as its single-pass kernel
(forward_onepass); with few (batch, head) pairs it adds a segment-state
kernel first (segment_states); shapes outside the single-pass kernel run
the stages chunk_cumsum, chunk_state, state_passing, chunk_cb, chunk_scan.
The library's own ssd_forward_plan says which.

Per-kernel GPU times come from HIP events the library records between its
launches (ssd_forward_timed) on the launch stream, inside the timed region.
Roofline figures use algorithmic bytes / flops (what the method must read,
write and compute), not executed ones. The decode step (256 x 80 heads,
P 64, N 128, fp32 state, 64 consecutive tokens) is reported alongside.
The CPU baseline is the fp64 oracle (test infrastructure) on the same
workload, timed on this host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--all] [--no-cpu]
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

def segments_of(w):
    """The library's own plan for this forward (ssd_forward_plan): S >= 1
    segments per sequence on the single-pass kernel, 0 for the stage kernels."""
    import torch
    import structured_state_space_ssd_amd as ssd
    return ssd.forward_plan(w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate, w.chunk,
                            torch.bfloat16 if w.dtype == "bf16" else torch.float32)


def onepass_path(w):
    """Whether the library runs this forward as its single-pass kernel."""
    return segments_of(w) > 0


def stages_of(w):
    S = segments_of(w)
    return STAGES if S == 0 else (ONEPASS if S == 1 else ONEPASS_SEG)


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
    states (float32 P x N per (batch, head, segment), 2NP flops per
    token-head), which the single-pass kernel reads back."""
    Bt, L, H, P, G, N = w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate
    T = 64
    tok = Bt * L
    S, k, per_seg = onepass_plan(w)
    seg_states = Bt * H * (S - 1) * k * (P * N + 1) * 4  # one state + decay per piece
    nbytes = 2 * tok * H * P * 2 + tok * H * 2 + 2 * tok * G * N * 2 + 2 * H * 4 + seg_states
    flops = tok * H * ((T + 1) * P + 4 * N * P + 2 * P) + tok * G * (T + 1) * N
    acc = {"forward_onepass": {"bytes": nbytes, "flops": flops}}
    if S > 1:
        pre = Bt * (S - 1) * per_seg * T  # tokens of the first S-1 segments
        acc["segment_states"] = {"bytes": pre * H * (P * 2 + 2) + pre * G * N * 2 + H * 4 +
                                          seg_states,
                                 "flops": pre * H * 2 * N * P}
    return acc


def onepass_plan(w):
    """(S, k, per_seg): segments, pieces per segment and blocks per segment of
    the single-pass forward, from the library's own plan (ssd_forward_plan_info)."""
    import torch
    import structured_state_space_ssd_amd as ssd
    p = ssd.plan_info(w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate, w.chunk,
                      torch.bfloat16 if w.dtype == "bf16" else torch.float32)
    assert p["path"] == "single_pass", p
    return p["segments"], max(1, p["pieces"]), p["segment_blocks"]


def accounting(w):
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
    chunk-head element pair.
    """
    if onepass_path(w):
        return onepass_accounting(w)
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
    if fused_state_path(w):
        # one kernel for stages 2 and 3 (the library's rule): reads x, B, s and
        # delta, writes chunk_init and the final state; no per-chunk states
        fin = Bt * H * P * N * 4
        state = {"bytes": x + bc + 2 * s + ci + fin,
                 "flops": state["flops"] + passing["flops"]}
        passing = {"bytes": 0, "flops": 0}
    acc = {
        "chunk_cumsum": cumsum,
        "chunk_state": state,
        "state_passing": passing,
        "chunk_cb": cb_stage,
        "chunk_scan": scan,
    }
    return acc


def fused_state_path(w):
    """Whether the library runs stages 2 and 3 as one kernel for this workload
    (bf16 with batch * nheads >= 512; mirrors state_passing_fused in the
    library's chunk_state.hip)."""
    return w.dtype == "bf16" and w.batch * w.nheads >= 512


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


def measured_traffic(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current source of the kernel; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(kernel)
    if not rec or rec.get("source_digest") != kernel_source_digest(kernel):
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------- GPU timing

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


def time_forward(w, steps, warmup, breakdown_steps=10, event_every=5, spin_seconds=0.15):
    """Two passes over the same resident inputs.

    Breakdown pass (not the timed region): ``breakdown_steps`` forwards with a
    HIP event between every two stages, giving each stage's GPU time (an event
    between launches also adds a small gap of its own).
    Timed region: ``warmup`` untimed forwards, then ``steps`` forwards between
    two synchronizations, timed by the host clock; inside it, events are
    recorded only around the dominant stage of the breakdown pass, on the
    launch stream, in every ``event_every``-th forward (an event pair costs a
    few microseconds of pipeline gap), so that the dominant kernel's average
    time is measured live with little added overhead."""
    import torch
    import ssd_workloads as W
    import structured_state_space_ssd_amd as ssd

    d = W.generate(w)
    g = upload(d)
    x, dt, A, B, C, D = (g[k] for k in ("x", "dt", "A", "B", "C", "D"))
    ws = torch.empty(ssd.workspace_size(w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate,
                                        w.chunk, x.dtype), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    stages = stages_of(w)
    ns = len(stages)  # events 0..ns used (the single-pass kernel: events 0 and 1)
    mk = lambda: torch.cuda.Event(enable_timing=True)
    pad = lambda evs: list(evs) + [None] * (len(STAGES) + 1 - len(evs))

    # ---- spin-up (see spin_up) before anything is measured
    spin_up(lambda: ssd.forward(x, dt, A, B, C, D, chunk=w.chunk, workspace=ws, y=y), spin_seconds)

    # ---- breakdown pass
    bd = [[mk() for _ in range(ns + 1)] for _ in range(breakdown_steps)]
    for evs in bd:
        ssd.forward(x, dt, A, B, C, D, chunk=w.chunk, workspace=ws, y=y, events=pad(evs))
    torch.cuda.synchronize()
    per_stage = [sum(evs[i].elapsed_time(evs[i + 1]) for evs in bd) / breakdown_steps
                 for i in range(ns)]
    evented_ms = sum(evs[0].elapsed_time(evs[ns]) for evs in bd) / breakdown_steps
    dom = max(range(ns), key=lambda i: per_stage[i])

    # ---- timed region
    sampled = list(range(0, steps, event_every))
    pairs = [(mk(), mk()) for _ in sampled]
    events = [None] * steps
    for k, (e0, e1) in zip(sampled, pairs):
        evs = [None] * (ns + 1)
        evs[dom], evs[dom + 1] = e0, e1
        for e in (e0, e1):
            e.record()  # create the HIP events before the timed region
        events[k] = pad(evs)
    for _ in range(warmup):
        ssd.forward(x, dt, A, B, C, D, chunk=w.chunk, workspace=ws, y=y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        ssd.forward(x, dt, A, B, C, D, chunk=w.chunk, workspace=ws, y=y, events=events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_ms = sum(e0.elapsed_time(e1) for e0, e1 in pairs) / len(pairs)
    return {"wall_ms": wall * 1e3 / steps, "evented_ms": evented_ms,
            "stage_ms": dict(zip(stages, per_stage)), "dominant": stages[dom], "dominant_ms": dom_ms}


def time_forward_cold(w, reps=30, flush_bytes=1 << 30):
    """Single forwards with nothing of the inputs in the caches: before each,
    outside its events, a 1 GiB buffer is read (a sum: clean lines only, so
    the forward does not also write back a flush's dirty lines), which leaves
    neither L2 nor the 256 MB Infinity Cache holding x, B, C or dt. The 2.7B
    inputs (175 MB) fit in the Infinity Cache, so back-to-back forwards (the
    timed region) find part of them there. Returns the median and p10 / p90
    in ms."""
    import torch
    import ssd_workloads as W
    import structured_state_space_ssd_amd as ssd

    g = upload(W.generate(w))
    x, dt, A, B, C, D = (g[k] for k in ("x", "dt", "A", "B", "C", "D"))
    ws = torch.empty(ssd.workspace_size(w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate,
                                        w.chunk, x.dtype), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    flush = torch.ones(flush_bytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros((), dtype=torch.float32, device="cuda")
    call = lambda: ssd.forward(x, dt, A, B, C, D, chunk=w.chunk, workspace=ws, y=y)
    spin_up(call)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for e0, e1 in evs:
        sink += flush.sum()
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    return {"median_ms": t[reps // 2], "p10_ms": t[reps // 10], "p90_ms": t[(9 * reps) // 10]}


def time_forward_options(w, steps, warmup):
    """Whole-forward time (host clock, no events, after spin_up) with every
    step-size option on: per-head bias, softplus, clamp to [4e-3, 3e-2] and the zero-order-hold
    input weight, on the same shapes (raw dt from generate_dt_raw)."""
    import torch
    import ssd_workloads as W
    import structured_state_space_ssd_amd as ssd

    d = W.generate(w)
    r = W.generate_dt_raw(w)
    d["dt"], d["dt_bias"] = r["dt"], r["dt_bias"]
    g = upload(d)
    x = g["x"]
    ws = torch.empty(ssd.workspace_size(w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate,
                                        w.chunk, x.dtype), dtype=torch.uint8, device="cuda")
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
    g = upload(W.generate(w))
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


def time_backward(w, steps, warmup):
    """Whole-backward time (host clock): gradients of every input for the
    workload's forward, with a final-state gradient and every dt option off."""
    import torch
    import ssd_workloads as W
    import structured_state_space_ssd_amd as ssd

    d = W.generate(w)
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
    t0 = time.perf_counter()
    for _ in range(steps):
        ssd.backward(*args, **kw)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


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
    import ssd_workloads as W
    d = W.generate(w)
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


def counters_run(w):
    """A short, fixed sequence of launches for counter collection."""
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
    time_forward(w, steps=3, warmup=1)
    print("[counters] forward x4 done", file=sys.stderr, flush=True)
    time_decode(W_decode(), warmup=0)
    print("[counters] decode done", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- profile summaries
#
# The rocprofv3 runs these read (OUT is any scratch directory):
TRACE_CMD = ('rocprofv3 --kernel-trace --stats --output-format csv -d "$OUT/trace" -o trace '
             '-- python bench.py --steps 20 --warmup 5 --all > "$OUT/bench_trace.log"')
FETCH_CMD = ('rocprofv3 --pmc FETCH_SIZE --output-format csv -d "$OUT/fetch" -o fetch '
             '-- python bench.py --counters')
WRITE_CMD = ('rocprofv3 --pmc WRITE_SIZE --output-format csv -d "$OUT/write" -o write '
             '-- python bench.py --counters')
# kernel-name fragment -> stage, first match wins (the fused stage-2+3 kernel
# fills the chunk_state interval of the forward)
KERNEL_OF = {"segment_states_kernel": "segment_states",
             "ssd_forward_onepass": "forward_onepass", "onepass_varlen_prep": "packed: token int4s",
             "chunk_cumsum_kernel": "chunk_cumsum", "chunk_state_passing": "chunk_state",
             "state_passing_kernel": "state_passing", "chunk_state": "chunk_state",
             "chunk_cb_kernel": "chunk_cb", "chunk_scan": "chunk_scan",
             "decode_step_kernel": "decode_step", "chunk_bwd_kernel": "backward: chunk gradients",
             "bwd_dt_kernel": "backward: dt, A, bias", "bwd_reduce_kernel": "backward: dB, dC sums",
             "bwd_head_sum_kernel": "backward: per-head sums", "varlen_seg": "packed: token masks"}
UTIL_CMDS = ('rocprofv3 --pmc MfmaUtil VALUBusy LdsUtil --output-format csv -d "$OUT/util" -o util '
             '-- python bench.py --counters',
             'rocprofv3 --pmc MfmaFlopsBF16 --output-format csv -d "$OUT/mops" -o mops '
             '-- python bench.py --counters')
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


def summarize_trace(stats_csv, bench_log):
    """Markdown table of a --kernel-trace --stats run, with the bench line's own
    event timings of the same run beside the profiler's averages."""
    rows = _read_csv(stats_csv)
    bench = None
    with open(bench_log) as f:
        for line in f:
            if line.startswith("{"):
                bench = json.loads(line)
    out = ["# Kernel trace: SSD forward stages (Mamba-2 2.7B-shaped layer) and decode step", "",
           "The same run also times the forward with every step-size option, the packed",
           "variable-length forward and the backward on the same shapes (bench.py's",
           "forward_with_options, forward_varlen and backward entries) and, with --all, the",
           "tiny, large-state and long-sequence forwards; their kernels are listed too. A",
           "kernel name can appear for several uses (e.g. the chunk-state kernel computes the",
           "backward's output-gradient contributions as well). The bench's own event time is",
           "given beside the 2.7B forward's kernel (the first row of its stage) only.", "",
           "Commands, from the repository root on one MI355X:", "", "```",
           "cd /tmp && export TMPDIR=/tmp && cd -", TRACE_CMD,
           f'python bench.py --summarize-trace "$OUT/trace/trace_kernel_stats.csv" "$OUT/bench_trace.log"',
           "```", "",
           "| kernel | stage | calls | avg us | min us | max us | bench event avg us |",
           "|---|---|---|---|---|---|---|"]
    seen = set()
    for r in rows:
        stage = _stage_of(r["Name"])
        ev = ""
        if bench and stage in bench.get("kernels", {}) and stage not in seen:
            ev = f"{bench['kernels'][stage]['us']:.2f}"
            seen.add(stage)
        elif bench and stage == "decode_step":
            ev = f"{bench['decode']['us_per_step']:.2f}"
        name = r["Name"].split("(")[0].replace("void ", "")
        out.append(f"| `{name}` | {stage or '-'} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {ev} |")
    if bench:
        out += ["", f"Bench line of the same run: value {bench['value']:.4g} tokens/s, "
                    f"{bench['ms_per_step'] * 1e3:.1f} us per forward, roofline "
                    f"{json.dumps(bench['roofline'])}."]
    return "\n".join(out)


def summarize_traffic(fetch_csv, write_csv, workload="mamba2_2.7b"):
    """HBM bytes per launch of each kernel from FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch), each scaled by what the same counter reads for the
    plain 1 GiB device copy of the same run. Returns (markdown, json dict)."""
    import ssd_workloads as W
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
    acc = accounting(W.WORKLOADS[workload])
    acc["decode_step"] = decode_accounting(W_decode())
    rec = {"_calibration": {"kernel": CALIBRATION_KERNEL, "copy_bytes": COPY_BYTES,
                            "fetch_kib": max(cal["fetch"]), "write_kib": max(cal["write"]),
                            "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
                            "commands": [FETCH_CMD, WRITE_CMD]}}
    wopt = "" if workload == "mamba2_2.7b" else f" --workload {workload}"
    title = {"mamba2_2.7b": "Mamba-2 2.7B-shaped layer",
             "long_seq": "long sequence: batch 1, L 65536, 80 heads, N 128, 8 groups"}.get(
                 workload, workload)
    out = [f"# HBM traffic per launch: SSD forward kernels ({title}) and decode step",
           "", "Commands, from the repository root on one MI355X:", "", "```",
           "cd /tmp && export TMPDIR=/tmp && cd -", f"timeout -s KILL 60 {FETCH_CMD}{wopt}",
           f"timeout -s KILL 60 {WRITE_CMD}{wopt}",
           'python bench.py --summarize-traffic "$OUT/fetch/fetch_counter_collection.csv" '
           f'"$OUT/write/write_counter_collection.csv"{wopt}', "```", "",
           f"Calibration: the 1 GiB device copy reads FETCH_SIZE {max(cal['fetch']):.0f} KiB and "
           f"WRITE_SIZE {max(cal['write']):.0f} KiB, so FETCH_SIZE is scaled by {f_scale:.3f} and "
           f"WRITE_SIZE by {w_scale:.3f}.", "",
           "| kernel | dispatches | fetch MB | write MB | HBM MB / launch | algorithmic MB | ratio |",
           "|---|---|---|---|---|---|---|"]
    for k in ONEPASS_SEG + STAGES + ["decode_step"]:
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
    bf16 MFMA flops against the algorithmic ones, per forward kernel."""
    import ssd_workloads as W
    per = {}
    for path in (util_csv, mops_csv):
        for r in _read_csv(path):
            k = _stage_of(r["Kernel_Name"])
            if k is None:
                continue
            per.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    acc = accounting(W.WORKLOADS[workload])
    wopt = "" if workload == "mamba2_2.7b" else f" --workload {workload}"
    out = [f"# MFMA, VALU and LDS utilisation: SSD forward kernels ({workload})", "",
           "rocprofv3 derived counters, each the average over the kernel's dispatches:",
           "MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs), VALUBusy and",
           "LdsUtil likewise in percent of busy cycles; MfmaFlopsBF16 = 512 x",
           "SQ_INSTS_VALU_MFMA_MOPS_BF16, the executed bf16 MFMA flops per launch, beside",
           "the algorithmic flops the accounting counts (the executed ones include the",
           "zero-padded halves of causal tiles and the D x products).", "",
           "Commands, from the repository root on one MI355X:", "", "```",
           "cd /tmp && export TMPDIR=/tmp && cd -"] + \
          [f"timeout -s KILL 60 {c}{wopt}" for c in UTIL_CMDS] + \
          ['python bench.py --summarize-util "$OUT/util/util_counter_collection.csv" '
           f'"$OUT/mops/mops_counter_collection.csv"{wopt}', "```", "",
           "| kernel | dispatches | MfmaUtil % | VALUBusy % | LdsUtil % | executed MFMA GFLOP "
           "| algorithmic GFLOP |", "|---|---|---|---|---|---|---|"]
    avg = lambda v: sum(v) / len(v) if v else float("nan")
    for k in ONEPASS_SEG + STAGES:
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="mamba2_2.7b")
    ap.add_argument("--all", action="store_true", help="also time the other forward workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--counters", action="store_true",
                    help="short run for rocprofv3 counter collection: a few forwards, a few decode "
                         "steps and a plain 1 GiB device copy that calibrates the byte counters")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("STATS_CSV", "BENCH_LOG"),
                    help="print the markdown summary of a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--summarize-util", nargs=2, metavar=("UTIL_CSV", "MOPS_CSV"),
                    help="print the MFMA / VALU / LDS utilisation summary of two rocprofv3 "
                         "--pmc runs")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM-traffic summary of two rocprofv3 --pmc runs and write "
                         "profiles/hbm_traffic.json")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(*args.summarize_trace))
        return
    if args.summarize_util:
        print(summarize_util(*args.summarize_util, workload=args.workload))
        return
    if args.summarize_traffic:
        md, rec = summarize_traffic(*args.summarize_traffic, workload=args.workload)
        if args.workload == "mamba2_2.7b":  # the bench line's roofline.traffic reads this one
            with open(TRAFFIC_FILE, "w") as f:
                json.dump(rec, f, indent=1)
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
        counters_run(w)
        return
    print(f"[bench] {w.name}: timing {args.steps} steps after {args.warmup} warmup", file=sys.stderr, flush=True)
    fwd = time_forward(w, args.steps, args.warmup)
    ms = fwd["wall_ms"]
    acc = accounting(w)
    kernels = {}
    for name in stages_of(w):
        t = fwd["stage_ms"][name] * 1e-3
        a = acc[name]
        if a["bytes"] == 0:  # stage not launched for this dtype (only event gaps in between)
            kernels[name] = {"us": round(t * 1e6, 2), "launched": False}
            continue
        gbs = a["bytes"] / t / 1e9
        tfl = a["flops"] / t / 1e12
        peak_f = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
        intensity = a["flops"] / a["bytes"]
        applicable = min(peak_f, intensity * HBM_PEAK_GBS / 1e3)  # TFLOP/s roof at this intensity
        kernels[name] = {"us": round(t * 1e6, 2), "alg_bytes": a["bytes"], "alg_flops": a["flops"],
                         "GB_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                         "TFLOP_s": round(tfl, 2), "mfma_frac": round(tfl / peak_f, 4),
                         "roofline_frac": round(tfl / applicable, 4)}
    dom = fwd["dominant"]
    dom_gbs = acc[dom]["bytes"] / (fwd["dominant_ms"] * 1e-3) / 1e9  # live, in the timed region
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                "us_per_launch": round(fwd["dominant_ms"] * 1e3, 2),
                "traffic": measured_traffic(dom)}
    print(f"[bench] forward {ms * 1e3:.1f} us/step ({fwd['evented_ms'] * 1e3:.1f} us with an event "
          f"between every two kernels; {fwd['dominant']} {fwd['dominant_ms'] * 1e3:.1f} us live); kernels " +
          ", ".join(f"{k} {v['us']:.1f} us" for k, v in kernels.items()), file=sys.stderr, flush=True)

    cold = time_forward_cold(w)
    cold_rec = {"protocol": "one forward per rep after reading a 1 GiB buffer (L2 and Infinity "
                            "Cache hold none of the inputs); 30 reps",
                "us_per_forward": round(cold["median_ms"] * 1e3, 2),
                "p10_us": round(cold["p10_ms"] * 1e3, 2), "p90_us": round(cold["p90_ms"] * 1e3, 2),
                "tokens_per_s": round(w.tokens / (cold["median_ms"] * 1e-3), 1)}
    print(f"[bench] cold-cache forward: {cold_rec['us_per_forward']} us (median)", file=sys.stderr,
          flush=True)

    opt_ms = time_forward_options(w, max(10, args.steps // 2), 3)
    options = {"options": "dt_bias + softplus + clamp + zero-order hold",
               "us_per_forward": round(opt_ms * 1e3, 2),
               "tokens_per_s": round(w.tokens / (opt_ms * 1e-3), 1)}
    print(f"[bench] forward with every step-size option: {opt_ms * 1e3:.1f} us", file=sys.stderr,
          flush=True)

    wv, cu, vl_ms = time_forward_varlen(max(10, args.steps // 2), 3)
    varlen = {"workload": f"{wv.seqlen} tokens (the 2.7B layer's 8 x 2048) packed as {cu.size - 1} "
                          "sequences of 1 .. 4096 tokens, bf16, per-sequence final states",
              "us_per_forward": round(vl_ms * 1e3, 2),
              "tokens_per_s": round(wv.seqlen / (vl_ms * 1e-3), 1)}
    print(f"[bench] packed variable-length forward: {vl_ms * 1e3:.1f} us", file=sys.stderr,
          flush=True)

    bw_ms = time_backward(w, max(10, args.steps // 2), 3)
    backward = {"workload": "gradients of x, dt, A, B, C, D and the initial state, same shapes",
                "us_per_backward": round(bw_ms * 1e3, 2),
                "tokens_per_s": round(w.tokens / (bw_ms * 1e-3), 1)}
    print(f"[bench] backward: {bw_ms * 1e3:.1f} us", file=sys.stderr, flush=True)

    extra = {}
    if args.all:
        for name in ("tiny_f32", "large_state", "long_seq"):
            wl = W.WORKLOADS[name]
            r = time_forward(wl, 10, 3)
            acc_w = accounting(wl)
            hbm = {}
            for k, v in r["stage_ms"].items():
                nb, nf = acc_w[k]["bytes"], acc_w[k]["flops"]
                if nb and v > 0:
                    gbs = nb / (v * 1e-3) / 1e9
                    tfl = nf / (v * 1e-3) / 1e12
                    peak = BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_PEAK_TFLOPS
                    hbm[k] = {"alg_MB": round(nb / 1e6, 1), "GB_s": round(gbs, 1),
                              "hbm_frac": round(gbs / HBM_PEAK_GBS, 3),
                              "TFLOP_s": round(tfl, 2), "mfma_frac": round(tfl / peak, 4)}
            extra[name] = {"us_per_forward": round(r["wall_ms"] * 1e3, 1),
                           "tokens_per_s": round(wl.tokens / (r["wall_ms"] * 1e-3)),
                           "stage_us": {k: round(v * 1e3, 1) for k, v in r["stage_ms"].items()},
                           "stage_hbm": hbm}
            print(f"[bench] {name}: {r['wall_ms'] * 1e3:.1f} us", file=sys.stderr, flush=True)

    wd = W.WORKLOADS["decode"]
    dec = time_decode(wd)
    da = decode_accounting(wd)
    dec_gbs = da["bytes"] / (dec["mean_ms"] * 1e-3) / 1e9
    decode = {"workload": "decode: batch 256, 80 heads x P 64, N 128, fp32 state, bf16 inputs, 64 steps",
              "us_per_step": round(dec["mean_ms"] * 1e3, 2), "GB_s": round(dec_gbs, 1),
              "hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4), "alg_bytes_per_step": da["bytes"],
              "tokens_per_s": round(wd.batch / (dec["mean_ms"] * 1e-3))}
    print(f"[bench] decode {decode['us_per_step']} us/step, {decode['GB_s']} GB/s", file=sys.stderr, flush=True)

    probe = hbm_probe()
    print(f"[bench] 1 GiB device copy: {probe['read_plus_write_GB_s']} GB/s (read + write)",
          file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu:
        print("[bench] cpu baseline (fp64 oracle)...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w)

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
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "evented_us_per_step": round(fwd["evented_ms"] * 1e3, 2),
        "kernels": kernels,
        "forward_cold_cache": cold_rec,
        "forward_with_options": options,
        "forward_varlen": varlen,
        "backward": backward,
        "decode": decode,
        "hbm_copy_probe": probe,
    }
    if extra:
        out["other_workloads"] = extra
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
