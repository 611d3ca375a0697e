"""The seeded input generator: determinism, block independence, bf16 rounding."""
import numpy as np
import torch

import ttt_inputs as ti


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 10000),
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -9, -1 - 2 ** -8, 0.0, -0.0], np.float32)]).astype(np.float32)
    vals, bits = ti.bf16_round(x)
    t = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(bits, t.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(vals, t.to(torch.float32).numpy())


def test_generation_is_deterministic_and_blockwise():
    cfg = ti.Config("g", 2, 2, 70000, 1000, 16, 32, act="bf16", seed=77)
    a = ti.make_problem_inputs(cfg, 1, 0)
    b = ti.make_problem_inputs(cfg, 1, 0)
    for k in a:
        assert np.array_equal(a[k], b[k])
    part = ti.make_problem_inputs(cfg, 1, 0, t0=65000, t1=66000)
    for k in ("q", "k", "v", "eta"):
        assert np.array_equal(part[k], a[k][65000:66000])
    other = ti.make_problem_inputs(cfg, 0, 1)
    assert not np.array_equal(other["q"], a["q"])


def test_distributions():
    cfg = ti.Config("g", 1, 1, 4096, 512, 64, 128, act="bf16", seed=5)
    p = ti.make_problem_inputs(cfg, 0, 0)
    n = np.linalg.norm(p["q"].astype(np.float64), axis=1)
    assert np.abs(n - 1).max() < 1e-2          # unit norm up to bf16 rounding
    assert 0.0 < p["eta"].min() and p["eta"].max() < 0.01
    assert abs(p["eta"].mean() - 0.005) < 3e-4
    assert abs(p["v"].std() - 1) < 0.02
    w = ti.make_weights(cfg)
    assert w[0].shape == (1, 128, 64) and w[2].shape == (1, 64, 128)
    assert abs(w[0].std() - 64 ** -0.5) < 0.01
    vals, _ = ti.bf16_round(p["k"])
    assert np.array_equal(vals, p["k"])        # already bf16 values


def test_full_tensor_matches_problem_slices():
    cfg = ti.Config("g", 2, 3, 300, 100, 16, 32, act="f32", seed=3)
    full = ti.make_inputs(cfg)
    p = ti.make_problem_inputs(cfg, 1, 2)
    assert np.array_equal(full["v"][1, 2], p["v"])
    assert full["q"].shape == (2, 3, 300, 16) and full["eta"].shape == (2, 3, 300)
