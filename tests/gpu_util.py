"""Helpers shared by the GPU tests: upload generated inputs, run the oracle,
compare. Relative L2 = ||gpu - ref||_2 / ||ref||_2 over the flattened tensor,
in float64."""
import numpy as np

import ssd_workloads as W

TOL_F32 = 1e-4   # relative L2 for float32 inputs
TOL_BF16 = 2e-2  # relative L2 for bf16 inputs
TOL_DECODE_STATE = 1e-3


def tol(dtype):
    return TOL_F32 if dtype == "f32" else TOL_BF16


def up(t, dev="cuda"):
    import torch
    if t is None:
        return None
    if isinstance(t, W.Tensor):
        if t.dtype == "bf16":
            return torch.from_numpy(t.dev.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(t.dev).to(dev)
    return torch.from_numpy(np.ascontiguousarray(t)).to(dev)


def down(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def rel_l2(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def unit_rel_l2(a, b, part=None):
    """Relative L2 of each unit (leading axis) of a against b: an array of
    ||a_u - b_u|| / ||b_u||, in float64 (a unit whose reference is all zero
    gives ||a_u||). Each head's semiseparable matrix is an independent unit of
    the computation, so a wrong unit shows here even when the whole-tensor
    norm would hide it.

    ``part`` (optional, same shape as b): one of two terms that b is the sum
    of (y = state-space part + D x); the denominator is then the larger of
    ||b_u|| and ||part_u||. A unit whose two terms nearly cancel (a head with
    D close to minus the state-space gain, over a one-token sequence) has a
    tiny ||b_u||, and the rounding of each term, which both sides take in
    their own precision, is measured against the terms' own size."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    a = a.reshape(a.shape[0], -1)
    b = b.reshape(b.shape[0], -1)
    den = np.linalg.norm(b, axis=1)
    if part is not None:
        den = np.maximum(den, np.linalg.norm(np.asarray(part, np.float64).reshape(b.shape), axis=1))
    return np.linalg.norm(a - b, axis=1) / np.where(den > 0, den, 1.0)


def check_units(name, a, b, t, labels=None, part=None):
    """Assert every unit's relative L2 (unit_rel_l2) below t; print the worst
    unit. Returns the worst error."""
    e = unit_rel_l2(a, b, part)
    if e.size == 0:
        return 0.0
    k = int(np.argmax(e))
    lab = labels[k] if labels is not None else k
    print(f"   per-unit {name}: worst {e[k]:.3e} at unit {lab} of {e.size}, median "
          f"{float(np.median(e)):.3e}", flush=True)
    assert e[k] < t, (name, lab, float(e[k]))
    return float(e[k])


def units_view(y_bthp, units, H):
    """Gather [U, L, P] from y [Bt, L, H, P] for flat units b*H + h."""
    u = np.asarray(units)
    return y_bthp[u // H, :, u % H, :]


def print_case(msg):
    print(msg, flush=True)
