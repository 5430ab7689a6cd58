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


def units_view(y_bthp, units, H):
    """Gather [U, L, P] from y [Bt, L, H, P] for flat units b*H + h."""
    u = np.asarray(units)
    return y_bthp[u // H, :, u % H, :]


def print_case(msg):
    print(msg, flush=True)
