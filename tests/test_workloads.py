"""The seeded input generator: rounding, determinism, shapes, distributions."""
import math

import numpy as np

import ssd_workloads as W


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.00390625, 1.005859375, 1.01171875, -2.5, 3.0e-39, 65504.0], np.float32)
    bits = W.f32_to_bf16_bits(vals)
    back = W.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0)
    assert back[1] == 1.0
    # 1 + 1.5*2^-8 rounds up to 1 + 2^-7
    assert back[2] == np.float32(1.0078125)
    assert back[0] == 1.0 and back[4] == -2.5
    rng = np.random.default_rng(0)
    r = rng.standard_normal(100000).astype(np.float32)
    rb = W.bf16_bits_to_f32(W.f32_to_bf16_bits(r))
    assert np.max(np.abs(rb - r) / np.abs(r)) <= 2.0 ** -8  # half an ulp of an 8-bit significand
    # rounding is idempotent
    assert np.array_equal(W.f32_to_bf16_bits(rb), W.f32_to_bf16_bits(r))


def test_generate_is_deterministic_and_shaped():
    w = W.small("g", 2, 50, 4, 8, 2, 16, 16, "bf16", seed=3, init_std=0.1)
    a, b = W.generate(w), W.generate(w)
    for k in ("x", "B", "C", "dt"):
        assert np.array_equal(a[k].dev, b[k].dev)
        assert a[k].dev.dtype == np.uint16
    assert a["x"].shape == (2, 50, 4, 8) and a["B"].shape == (2, 50, 2, 16)
    assert a["dt"].shape == (2, 50, 4) and a["A"].shape == (4,) and a["init"].shape == (2, 4, 8, 16)
    c = W.generate(w, seed=4)
    assert not np.array_equal(a["x"].dev, c["x"].dev)


def test_distributions_match_recipe():
    w = W.small("d", 4, 2000, 16, 16, 1, 64, 64, "f32", seed=5)
    d = W.generate(w)
    assert abs(d["x"].val.std() - 1.0) < 0.01
    assert abs(d["B"].val.std() - 1 / 8) < 0.002
    dt = d["dt"].val
    assert dt.min() >= 1e-3 * (1 - 1e-6) and dt.max() <= 1e-1 * (1 + 1e-6)
    ld = np.log(dt)
    assert abs(ld.mean() - 0.5 * (math.log(1e-3) + math.log(1e-1))) < 0.02
    A = d["A"]
    assert (A < 0).all() and (A >= -16).all() and (A <= -1).all()


def test_named_workloads():
    c1 = W.WORKLOADS["mamba2_2.7b"]
    assert (c1.batch, c1.seqlen, c1.nheads, c1.headdim, c1.dstate, c1.chunk) == (8, 2048, 80, 64, 64, 256)
    assert c1.nchunks == 8
    c3 = W.WORKLOADS["long_seq"]
    assert c3.ngroups == 8 and c3.nchunks == 256
    dec = W.WORKLOADS["decode"]
    assert dec.decode and dec.init_std == 0.1
