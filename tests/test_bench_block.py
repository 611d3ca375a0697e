"""bench.py's block mode: its flop accounting of the attention counts exactly the (query,
key) pairs the windows allow (brute force over the masks on small sequences)."""
import numpy as np
import pytest

import bench
import oracle.ttt_block as blk
import ttt_inputs as ti


@pytest.mark.parametrize("T,window,mode", [(100, 7, "sliding"), (100, 100, "sliding"),
                                           (100, 300, "sliding"), (100, 7, "block"),
                                           (100, 100, "block"), (96, 32, "block")])
def test_attention_pairs(T, window, mode):
    cfg = ti.Config("x", 2, 2, T, T, 128, 256, "swiglu", "dot", 5, True, "bf16")
    f = bench.block_part_flops(cfg, 256, 1024, window, mode)
    pairs = int(blk.window_mask(T, window, mode).sum())
    assert f["attention"] == 4.0 * 128 * pairs * 2 * 2
    assert f["proj_qkv"] == 2 * 2.0 * 2 * T * 256 * 768
    assert f["ffn_up"] == f["ffn_down"] == 2.0 * 2 * T * 256 * 1024
