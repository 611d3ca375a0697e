"""The stored image-set expectations cover what the GPU kernels tile: two whole rows from
every 128-row tile of every fast-weight matrix (a whole row spans every column tile, so
every 128 x 128 tile of a matrix and of its transpose holds compared values), and output
tokens from every 65536-token apply block, its first and last token among them."""
import os

import numpy as np

import ttt_inputs as ti

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "imageset_oracle.npz")


def test_golden_covers_every_weight_tile():
    g = np.load(GOLDEN)
    cfg = ti.CONFIGS["imageset"]
    for m, (rows, cols) in enumerate(cfg.matrix_shapes()):
        r = g[f"W{m}_rows"]
        assert g[f"W{m}"].shape == (len(r), cols)
        counts = np.bincount(r // 128, minlength=(rows + 127) // 128)
        assert len(counts) == (rows + 127) // 128 and counts.min() >= 2, (m, counts)
        assert g[f"W{m}_rownorm"].shape == (rows,)


def test_golden_covers_every_apply_block():
    g = np.load(GOLDEN)
    T = ti.CONFIGS["imageset"].seq_len
    tok = g["tokens"]
    assert g["O"].shape == (len(tok), ti.CONFIGS["imageset"].dim)
    for b0 in range(0, T, 65536):
        b1 = min(T, b0 + 65536)
        sel = tok[(tok >= b0) & (tok < b1)]
        assert b0 in sel and b1 - 1 in sel
        assert len(np.unique(sel // 128)) >= 16, b0
