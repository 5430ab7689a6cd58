"""The fp64 oracle against its pins (closed forms, the dual quadratic form,
invariants and a hand-worked example), plus the chunk-cumsum definition."""
import numpy as np
import pytest

import oracle
import ssd_workloads as W
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_chunk_cumsum_definition():
    """s_t restarts at every chunk start; with dt*A constant it is linear in
    the offset within the chunk, and a ragged last chunk is handled."""
    Bt, L, H, Q = 2, 70, 3, 16
    dt = np.full((Bt, L, H), 0.5, np.float32)
    A = np.array([-1.0, -2.0, -0.25], np.float32)
    s = oracle.chunk_cumsum(dt, A, Q)
    off = (np.arange(L) % Q) + 1
    expect = 0.5 * A[None, :, None].astype(np.float64) * off[None, None, :]
    assert np.allclose(s, np.broadcast_to(expect, s.shape), rtol=0, atol=1e-15)


def test_chunk_cumsum_vs_recurrence_decay():
    """exp of the chunk total equals the product of the per-token decays the
    recurrence applies, read from a zero-input run with an identity-like state."""
    w = W.small("cc", 1, 40, 2, 1, 1, 1, 16, "f32", seed=21)
    d = W.generate(w)
    dt, A = d["dt"].val, d["A"]
    s = oracle.chunk_cumsum(dt, A, 16)
    x = np.zeros((1, 40, 2, 1), np.float32)
    B = np.zeros((1, 40, 1, 1), np.float32)
    C = np.ones((1, 40, 1, 1), np.float32)
    init = np.ones((1, 2, 1, 1))
    # chunk 1 covers tokens 16..31: decay over the chunk = state(31) / state(15)
    _, _, snaps = oracle.forward(x, dt, A, B, C, None, init, snap_every=16)
    ratio = snaps[:, 1, 0, 0] / snaps[:, 0, 0, 0]
    assert np.allclose(ratio, np.exp(s[0, :, 31]), rtol=1e-13)


def test_oracle_units_subset_matches_full():
    w = W.small("units", 2, 33, 5, 4, 1, 6, 8, "f32", seed=22, init_std=0.1)
    d = W.generate(w)
    v = {k: (t.val if isinstance(t, W.Tensor) else t) for k, t in d.items()}
    y, st, _ = oracle.forward(v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], v["init"])
    units = [7, 0, 9]
    ys, sts, _ = oracle.forward(v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], v["init"], units=units)
    assert np.array_equal(ys, y[units]) and np.array_equal(sts, st[units])
    # thread count does not change the (per-unit sequential) result
    y1, _, _ = oracle.forward(v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], v["init"], nthreads=1)
    assert np.array_equal(y1, y)


def test_oracle_rejects_bad_shapes():
    x = np.zeros((1, 4, 3, 2), np.float32)
    dt = np.zeros((1, 4, 3), np.float32)
    B = np.zeros((1, 4, 2, 2), np.float32)  # 3 heads not divisible by 2 groups
    with pytest.raises(RuntimeError):
        oracle.forward(x, dt, np.zeros(3, np.float32), B, B, None)
