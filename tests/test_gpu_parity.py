"""GPU parity: libttt against the fp64 oracle on the same seeded inputs.

Tolerances (max relative error, per tensor: |x - y|_inf / |y|_inf, on the outputs O and on
every final fast-weight matrix): 1e-4 for fp32 activations, 2e-2 for bf16 activations with
fp32 accumulation. Sizes span several tiles in every dimension and end in ragged tails."""
import numpy as np
import pytest
import torch

import ttt_inputs as ti
import weight_sequence_layers_amd as W
from ttt_gpu import device_inputs, parity, read_state, rel_err, run_gpu, small

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _check(cfg, planes=None, problems=None, chunked=False, tol=None):
    inp = ti.make_inputs(cfg)
    O, Ws = run_gpu(cfg, inp, planes, chunked)
    eo, ew = parity(cfg, inp, O, Ws, problems)
    tol = TOL[cfg.act] if tol is None else tol
    print(f"{cfg.name}: O {eo:.3e} W {[f'{e:.3e}' for e in ew]} (tol {tol})", flush=True)
    assert eo <= tol and max(ew) <= tol, (eo, ew)
    return eo, ew


def test_tiny_fp32_full_size():
    _check(ti.CONFIGS["tiny"])


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("fw,loss,ns,renorm", [
    ("swiglu", "dot", 5, True), ("swiglu", "dot", 0, True), ("swiglu", "mse", 0, False),
    ("gelu", "mse", 0, False), ("gelu", "dot", 5, True), ("linear", "dot", 0, False),
    ("linear", "mse", 0, True),
])
def test_ragged_shapes(act, fw, loss, ns, renorm):
    cfg = ti.Config("ragged", 2, 3, 900, 300, 80, 176, fw, loss, ns, renorm, act,
                    "apply_then_update", 2024)
    _check(cfg)


@pytest.mark.parametrize("order", ["apply_then_update", "update_then_apply"])
def test_orders(order):
    cfg = ti.Config("ord", 1, 2, 1024, 256, 64, 128, "swiglu", "dot", 5, True, "bf16", order, 7)
    _check(cfg, planes=(1, 2, 2, 0))


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_token_split_contraction(act):
    # few output tiles and 1000-token chunks: the gradient contraction splits each chunk's
    # tokens into ranges of 384, 384 and 232 summed by a second pass (ragged last range)
    cfg = ti.Config("split", 1, 2, 2000, 1000, 64, 128, "swiglu", "dot", 5, True, act,
                    "apply_then_update", 31)
    _check(cfg)


def test_fp32_activations_two_gradient_planes():
    # fp32 keys and values split into two bf16 planes against two-plane errors: the token
    # contraction runs 2 x 2 planes plane-resident (three products a K step). The apply
    # uses one plane, so the bar is the bf16 one.
    cfg = ti.Config("f32p2", 2, 2, 600, 200, 80, 176, "swiglu", "dot", 5, True, "f32",
                    "apply_then_update", 81)
    _check(cfg, planes=(1, 2, 2, 0), tol=TOL["bf16"])


def test_wide_tiles_ragged_edges():
    # 30 (batch, head) problems at dim 144, hidden 288: enough matrices that the Gram,
    # polynomial and update stages take their 128-wide tiles, whose second tile row and
    # column hold only 16 of 144 rows (and the hidden tiles 32 of 128)
    cfg = ti.Config("wide", 10, 3, 256, 128, 144, 288, "swiglu", "dot", 5, True, "bf16",
                    "apply_then_update", 41)
    _check(cfg, planes=(1, 2, 2, 0), problems=[(0, 0), (4, 1), (9, 2)])


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("fw,loss,ns,renorm,lr,wd", [
    ("swiglu", "dot", 5, True, (0.5, 1.5, 0.8), 0.05),
    ("swiglu", "mse", 0, False, (0.7, 0.4, 1.3), 0.1),
    ("gelu", "mse", 0, False, (0.6, 1.7), 0.02),
    ("linear", "dot", 0, False, (0.3,), 0.2),
])
def test_step_size_and_weight_decay(act, fw, loss, ns, renorm, lr, wd):
    # per-matrix step sizes and a weight decay: W <- (1 - wd) W - lr_i U, then the renorm
    cfg = ti.Config("step", 2, 2, 600, 200, 80, 176, fw, loss, ns, renorm, act,
                    "apply_then_update", 77, lr=lr, weight_decay=wd)
    _check(cfg)


@pytest.mark.parametrize("shape", ["narrow", "wide"])
def test_single_plane_newton_schulz_one_chunk(shape):
    # Newton-Schulz with one bf16 plane everywhere: the 64-wide symmetric kernels (two
    # K groups of four waves) for a few matrices, the 128-wide ones for many. One chunk,
    # so that the plain-bf16 rounding does not compound over chunks.
    if shape == "narrow":
        cfg = ti.Config("np1", 1, 2, 400, 400, 80, 176, "swiglu", "dot", 5, True, "bf16",
                        "apply_then_update", 51)
        problems = None
    else:
        cfg = ti.Config("np1w", 10, 3, 256, 256, 144, 288, "swiglu", "dot", 5, True, "bf16",
                        "apply_then_update", 52)
        problems = [(0, 0), (9, 2)]
    _check(cfg, planes=(1, 1, 1, 0), problems=problems)


@pytest.mark.parametrize("planes", [(1, 1, 1, 0), (1, 2, 2, 0b00011)])
def test_fused_small_newton_schulz_planes(planes):
    # matrices of 64 x 128 run every Newton-Schulz iteration in one workgroup: one bf16
    # plane everywhere, and two planes with iterations 0 and 1 on one plane (B without a I,
    # a X added from the iterate's two planes). One chunk, as the single-plane tests above.
    cfg = ti.Config("nss", 2, 2, 256, 256, 64, 128, "swiglu", "dot", 5, True, "bf16",
                    "apply_then_update", 71)
    _check(cfg, planes=planes)


@pytest.mark.parametrize("planes", [(2, 2, 2, 0), (3, 3, 3, 0)])
def test_small_plane_resident_products(planes):
    # launches too small to fill the GPU (fp32 activations, dim 64) with the same number of
    # bf16 planes on every operand: the query and key-row fronts and the query output take
    # the plane-resident products (all plane tiles of a K step loaded once). Two planes are
    # held to the bf16 bar, three to the fp32 one.
    cfg = ti.Config("prf", 2, 1, 1024, 512, 64, 128, "swiglu", "dot", 0, True, "f32",
                    "apply_then_update", 91)
    _check(cfg, planes=planes, tol=2e-2 if planes[0] == 2 else 1e-4)


@pytest.mark.parametrize("case", ["two_blocks", "gelu_mse_f32"])
def test_fused_small_newton_schulz_after_split(case):
    # matrices of at most 64 x 128 (every Newton-Schulz iteration in one launch) after a
    # token-split contraction.
    # two_blocks: chunks of 66000 tokens, two token blocks each (the last block's split sum
    # also adds the first block's running sum); a step size per matrix, no renorm.
    # gelu_mse_f32: GELU net and MSE loss (two contraction launches), fp32 activations,
    # weight decay and renorm, dims off the tile grid.
    if case == "two_blocks":
        cfg = ti.Config("fss2", 1, 2, 132000, 66000, 64, 128, "swiglu", "dot", 5, False, "bf16",
                        "apply_then_update", 81, lr=(0.5, 1.0, 0.25))
        _check(cfg, planes=(1, 3, 3, 0))
    else:
        cfg = ti.Config("fssm", 3, 1, 8192, 4096, 48, 96, "gelu", "mse", 5, True, "f32",
                        "apply_then_update", 82, weight_decay=0.01)
        _check(cfg, planes=(3, 3, 3, 0))


@pytest.mark.parametrize("case", ["narrow_lead2", "narrow_all_one_chunk", "wide_lead2",
                                  "wide_mixed"])
def test_one_plane_newton_schulz_iterations(case):
    # Newton-Schulz iterations named in ns_one_plane multiply one bf16 plane and add the
    # linear term a X from the iterate's two stored planes; the others keep two planes.
    # Narrow: 12 matrices of 128 x 256 (64-wide tiles); wide: 90 matrices of 144 x 288
    # (128-wide tiles with ragged second rows and columns).
    if case.startswith("narrow"):
        one_chunk = case == "narrow_all_one_chunk"
        cfg = ti.Config("onep", 2, 2, 512 if one_chunk else 1024, 512 if one_chunk else 256,
                        128, 256, "swiglu", "dot", 5, True, "bf16", "apply_then_update", 61)
        mask, problems = (0b11111 if one_chunk else 0b00011), None
    else:
        cfg = ti.Config("onepw", 10, 3, 512, 128, 144, 288, "swiglu", "dot", 5, True, "bf16",
                        "apply_then_update", 62)
        mask, problems = (0b00011 if case == "wide_lead2" else 0b01010), [(0, 0), (9, 2)]
    _check(cfg, planes=(1, 2, 2, mask), problems=problems)


def _random_case(i):
    # seeded draw of a configuration: every net, loss, order, precision and the optional
    # Muon and renorm, with dims that are not tile multiples and chunks of any length
    rng = np.random.default_rng(900 + i)
    fw = ["swiglu", "gelu", "linear"][i % 3]
    loss = ["dot", "mse"][(i // 3) % 2]
    act = ["f32", "bf16"][(i // 2) % 2]
    dim = int(16 * rng.integers(1, 13))
    hidden = max(dim, int(16 * rng.integers(1, 21)))
    ns = 5 if (fw != "linear" and rng.random() < 0.6) else 0
    renorm = bool(rng.random() < 0.5)
    chunk = int(rng.integers(1, 300))
    n_chunks = int(rng.integers(1, 4))
    order = ["apply_then_update", "update_then_apply"][int(rng.integers(0, 2))]
    batch, heads = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    return ti.Config(f"rand{i}", batch, heads, chunk * n_chunks, chunk, dim, hidden, fw, loss,
                     ns, renorm, act, order, 3000 + i)


@pytest.mark.parametrize("i", range(12))
def test_random_shapes(i):
    cfg = _random_case(i)
    print(cfg, flush=True)
    _check(cfg)
