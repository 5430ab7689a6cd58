"""Seeded synthetic inputs for the SSD layer: shapes, distributions, seeds.

This module holds none of the SSD computation. It draws random tensors with
numpy and rounds them to their storage dtype; the oracle-side tests, the GPU
parity tests and the benchmark all read the same arrays from here.

Shapes follow the pages' models: the Mamba-2 2.7B configuration (d_model 2560,
expand 2 -> 80 heads of 64, state 64, sequence 2048; "Mamba-2架构深度解析",
section 3.1), the enlarged state N = 256 ("Mamba 模型", section 4.3), a long
sequence with grouped B/C heads, and recurrent (linear-mode) decode
("Mamba-2架构深度解析", section 2.2 table).

Conventions
-----------
* Draw order per workload is fixed: x, B, C, dt, A, D, init state.
* Values are drawn in float64 and rounded to float32 (round to nearest even);
  bf16 tensors are then rounded from float32 to bf16 (round to nearest even).
* Every tensor is returned twice: ``dev`` (the storage form handed to the GPU:
  ``np.uint16`` bf16 bit patterns or ``np.float32``) and ``val`` (``np.float32``
  holding exactly the same numbers, for the oracle).
* Large tensors are drawn in blocks; the generator stream makes the result the
  same as one draw of the whole tensor.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

_BLOCK = 1 << 24  # elements per generator call for large tensors


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int          # tokens per sequence (forward) or decode steps
    nheads: int
    headdim: int
    ngroups: int
    dstate: int
    chunk: int           # chunk length Q of the block decomposition (0: decode)
    dtype: str           # "f32" or "bf16": dtype of x, dt, B, C, y
    bc_scale: float      # B, C ~ N(0, 1) * bc_scale
    dt_lo: float         # dt = exp(U(ln dt_lo, ln dt_hi))
    dt_hi: float
    init_std: float = 0.0  # initial state ~ N(0, init_std); 0 means no init state
    decode: bool = False   # True: seqlen consecutive single-token steps
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def nchunks(self) -> int:
        return -(-self.seqlen // self.chunk) if self.chunk else 0

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32", 1, 256, 2, 64, 1, 16, 64, "f32", 1 / 4, 1e-3, 1e-1,
                 seed=1000, note="tiny fp32 forward"),
        Workload("mamba2_2.7b", 8, 2048, 80, 64, 1, 64, 256, "bf16", 1 / 8, 1e-3, 1e-1,
                 seed=1001, note="Mamba-2 2.7B-shaped layer, bf16"),
        Workload("large_state", 4, 4096, 32, 64, 1, 256, 128, "bf16", 1 / 16, 1e-3, 1e-1,
                 seed=1002, note="state N=256, bf16"),
        Workload("long_seq", 1, 65536, 80, 64, 8, 128, 256, "bf16", 1 / math.sqrt(128), 1e-4, 1e-2,
                 seed=1003, note="L=65536, 8 B/C groups, slow decay"),
        Workload("decode", 256, 64, 80, 64, 1, 128, 0, "bf16", 1 / math.sqrt(128), 1e-3, 1e-1,
                 init_std=0.1, decode=True, seed=1004, note="64 recurrent steps, fp32 state"),
    ]
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact float32 values of bf16 bit patterns."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


class Tensor:
    """A generated tensor: ``dev`` is the storage form, ``val`` the exact float32 values."""

    __slots__ = ("dev", "val", "dtype")

    def __init__(self, dev: np.ndarray, val: np.ndarray, dtype: str):
        self.dev, self.val, self.dtype = dev, val, dtype

    @property
    def shape(self):
        return self.val.shape


def _store(v32: np.ndarray, dtype: str) -> Tensor:
    if dtype == "bf16":
        bits = f32_to_bf16_bits(v32)
        return Tensor(bits, bf16_bits_to_f32(bits), "bf16")
    if dtype == "f32":
        v = np.ascontiguousarray(v32, dtype=np.float32)
        return Tensor(v, v, "f32")
    raise ValueError(f"unknown dtype {dtype}")


def _normal(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _BLOCK):
        e = min(n, s + _BLOCK)
        out[s:e] = rng.standard_normal(e - s) * scale
    return out.reshape(shape)


def _loguniform(rng: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _BLOCK):
        e = min(n, s + _BLOCK)
        out[s:e] = np.exp(rng.uniform(math.log(lo), math.log(hi), e - s))
    return out.reshape(shape)


def generate(w: Workload, seed: int | None = None) -> dict:
    """Draw the inputs of a workload.

    Forward workloads return x [Bt,L,H,P], dt [Bt,L,H], B and C [Bt,L,G,N]
    (all in ``w.dtype``), A and D [H] (float32) and ``init`` (float32
    [Bt,H,P,N] or None). Decode workloads put the step index first:
    x [T,Bt,H,P], dt [T,Bt,H], B and C [T,Bt,G,N], and ``init`` is the
    initial state.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    Bt, L, H, P, G, N = w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate
    if w.decode:
        sx, sd, sbc = (L, Bt, H, P), (L, Bt, H), (L, Bt, G, N)
    else:
        sx, sd, sbc = (Bt, L, H, P), (Bt, L, H), (Bt, L, G, N)
    out = {}
    out["x"] = _store(_normal(rng, sx), w.dtype)
    out["B"] = _store(_normal(rng, sbc, w.bc_scale), w.dtype)
    out["C"] = _store(_normal(rng, sbc, w.bc_scale), w.dtype)
    out["dt"] = _store(_loguniform(rng, sd, w.dt_lo, w.dt_hi), w.dtype)
    out["A"] = (-np.exp(rng.uniform(0.0, math.log(16.0), H))).astype(np.float32)
    out["D"] = rng.standard_normal(H).astype(np.float32)
    out["init"] = _normal(rng, (Bt, H, P, N), w.init_std) if w.init_std > 0 else None
    return out


def generate_dt_raw(w: Workload, seed: int | None = None) -> dict:
    """Inputs for the step-size preprocessing options: ``dt`` holds raw values
    (the step-size projection's output before its bias and softplus) drawn
    N(0, 0.5^2) and stored in ``w.dtype``, shaped like ``generate``'s dt;
    ``dt_bias`` is float32 [H] drawn U(-6.5, -2.5). softplus of their sum then
    spans roughly 2e-4 .. 0.3, the range of the plain workloads' dt. Drawn
    from a stream of its own, so ``generate``'s arrays are unchanged."""
    base = w.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(base + 0x5EED))
    Bt, L, H = w.batch, w.seqlen, w.nheads
    shape = (L, Bt, H) if w.decode else (Bt, L, H)
    return {"dt": _store(_normal(rng, shape, 0.5), w.dtype),
            "dt_bias": rng.uniform(-6.5, -2.5, H).astype(np.float32)}


def generate_grads(w: Workload, seed: int | None = None) -> dict:
    """Incoming gradients for the backward: dy ~ N(0, 1) shaped like x in
    ``w.dtype`` and dfinal ~ N(0, 1) float32 [Bt,H,P,N], from a stream of
    their own."""
    base = w.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(base + 0xB4C))
    Bt, L, H, P, N = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate
    return {"dy": _store(_normal(rng, (Bt, L, H, P)), w.dtype),
            "dfinal": _normal(rng, (Bt, H, P, N))}


def packed_cu_seqlens(total: int, max_len: int, seed: int) -> np.ndarray:
    """Offsets [nseq + 1] (int32, from 0 to total) of a packed batch of
    sequences with lengths floor(exp(U(0, ln(max_len + 1)))), i.e. spread
    log-uniformly over 1 .. max_len, the last one cut to fit: a mix of very
    short and long documents, as packing variable-length sequences produces."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cu = [0]
    while cu[-1] < total:
        n = max(1, int(np.exp(rng.uniform(0.0, math.log(max_len + 1)))))
        cu.append(min(total, cu[-1] + min(n, max_len)))
    return np.asarray(cu, dtype=np.int32)


def small(name: str, batch: int, seqlen: int, nheads: int, headdim: int, ngroups: int,
          dstate: int, chunk: int, dtype: str, seed: int, init_std: float = 0.0,
          dt_lo: float = 1e-3, dt_hi: float = 1e-1, bc_scale: float | None = None) -> Workload:
    """An ad-hoc forward workload with the same distributions as the named ones."""
    return Workload(name, batch, seqlen, nheads, headdim, ngroups, dstate, chunk, dtype,
                    bc_scale if bc_scale is not None else 1 / math.sqrt(dstate),
                    dt_lo, dt_hi, init_std=init_std, seed=seed)
