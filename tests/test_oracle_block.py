"""Pins of the block oracle (oracle/ttt_block.py): its window attention against torch's
scaled_dot_product_attention with the same boolean mask (a library routine), the window
masks against their definitions written as loops, RMS normalisation and the MLP against
torch, and the block's composition against its sub-layers called one by one."""
import numpy as np
import pytest
import torch

import oracle.ttt_block as blk
import oracle.ttt_oracle as orc
from ttt_inputs import Config


@pytest.mark.parametrize("mode,window", [("sliding", 5), ("sliding", 1), ("sliding", 40),
                                         ("block", 6), ("block", 40)])
def test_window_attention_matches_torch(mode, window):
    rng = np.random.default_rng(3)
    T, d = 23, 8
    Q, K, V = (rng.standard_normal((T, d)) for _ in range(3))
    ours = blk.window_attention(Q, K, V, window, mode)
    mask = torch.tensor(blk.window_mask(T, window, mode))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(Q)[None], torch.tensor(K)[None], torch.tensor(V)[None], attn_mask=mask[None])
    assert np.abs(ours - ref[0].numpy()).max() < 1e-12


def test_window_masks_match_their_definitions():
    T = 17
    for window in (1, 3, 4, 17, 30):
        m = blk.window_mask(T, window, "sliding")
        b = blk.window_mask(T, window, "block")
        for t in range(T):
            for j in range(T):
                assert m[t, j] == (t - window < j <= t)
                assert b[t, j] == (t // window == j // window)


def test_rmsnorm_and_mlp_match_torch():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((6, 16))
    ref = torch.nn.functional.rms_norm(torch.tensor(X), (16,), eps=blk.EPS).numpy()
    assert np.abs(blk.rmsnorm(X) - ref).max() < 1e-14
    w1, w2 = rng.standard_normal((32, 16)), rng.standard_normal((16, 32))
    t = torch.nn.functional.gelu(torch.tensor(X) @ torch.tensor(w1).T) @ torch.tensor(w2).T
    ours = blk.gelu(X @ w1.T) @ w2.T
    assert np.abs(ours - t.numpy()).max() < 1e-12


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(5).standard_normal(1000) * 10
    ref = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(blk.bf16(x), ref)


class _B:
    def __init__(self, ttt, window, mode):
        self.ttt, self.window, self.window_mode = ttt, window, mode


def test_block_is_its_sublayers_in_order():
    """y = h2 + mlp(n(h2)), h2 = h1 + ttt(n(h1)), h1 = x + attn(n(x)), each sub-layer called
    on its own here, the TTT heads through the sequence oracle directly."""
    rng = np.random.default_rng(6)
    D, T, H, d = 256, 64, 2, 128
    tcfg = Config("bt", 1, H, T, 32, d, 2 * d, "swiglu", "dot", 5, True, "bf16",
                  "apply_then_update", 1)
    b = _B(tcfg, 16, "sliding")
    w = {"attn_qkv": blk.bf16(rng.standard_normal((3 * D, D)) / 16),
         "attn_out": blk.bf16(rng.standard_normal((D, D)) / 16),
         "ttt_qkv": blk.bf16(rng.standard_normal((3 * D, D)) / 16),
         "ttt_eta": blk.bf16(rng.standard_normal((H, D)) / 16),
         "ttt_out": blk.bf16(rng.standard_normal((D, D)) / 16),
         "ffn_up": blk.bf16(rng.standard_normal((4 * D, D)) / 16),
         "ffn_down": blk.bf16(rng.standard_normal((D, 4 * D)) / 32)}
    W0 = [[rng.standard_normal(s) / np.sqrt(d) for s in tcfg.matrix_shapes()] for _ in range(H)]
    X = blk.bf16(rng.standard_normal((T, D)))
    y = blk.block_forward(b, w, X, W0)
    n = lambda a: blk.bf16(blk.rmsnorm(a))
    # attention by hand, per head
    qkv = blk.bf16(n(X) @ w["attn_qkv"].T)
    heads = []
    for h in range(D // 128):
        s = slice(h * 128, (h + 1) * 128)
        heads.append(blk.window_attention(qkv[:, s], qkv[:, D:][:, s], qkv[:, 2 * D:][:, s],
                                          16, "sliding"))
    h1 = blk.bf16(X + blk.bf16(np.concatenate(heads, 1)) @ w["attn_out"].T)
    # the TTT heads
    x2 = n(h1)
    qkv2 = blk.bf16(x2 @ w["ttt_qkv"].T)
    eta = (0.01 / (1 + np.exp(-(x2 @ w["ttt_eta"].T)))).astype(np.float32)
    outs = []
    for h in range(H):
        q = qkv2[:, h * d:(h + 1) * d]
        k = qkv2[:, D + h * d:D + (h + 1) * d]
        v = qkv2[:, 2 * D + h * d:2 * D + (h + 1) * d]
        q = blk.bf16(q / np.linalg.norm(q, axis=1, keepdims=True))
        k = blk.bf16(k / np.linalg.norm(k, axis=1, keepdims=True))
        O, _ = orc.sequence_forward(tcfg, W0[h], q, k, v, eta[:, h])
        outs.append(blk.bf16(O))
    h2 = blk.bf16(h1 + np.concatenate(outs, 1) @ w["ttt_out"].T)
    y_ref = blk.bf16(h2 + blk.bf16(blk.gelu(n(h2) @ w["ffn_up"].T)) @ w["ffn_down"].T)
    assert np.abs(y - y_ref).max() <= 1e-12 * np.abs(y_ref).max()


def test_window_special_cases():
    """Window 1 returns V itself; a sliding window covering the sequence is torch's causal
    attention; one block covering the sequence is full attention."""
    rng = np.random.default_rng(7)
    T, d = 19, 8
    Q, K, V = (rng.standard_normal((T, d)) for _ in range(3))
    assert np.abs(blk.window_attention(Q, K, V, 1, "sliding") - V).max() < 1e-14
    assert np.abs(blk.window_attention(Q, K, V, 1, "block") - V).max() < 1e-14
    t = [torch.tensor(a)[None] for a in (Q, K, V)]
    causal = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=True)[0].numpy()
    full = torch.nn.functional.scaled_dot_product_attention(*t)[0].numpy()
    assert np.abs(blk.window_attention(Q, K, V, T, "sliding") - causal).max() < 1e-12
    assert np.abs(blk.window_attention(Q, K, V, 1000, "sliding") - causal).max() < 1e-12
    assert np.abs(blk.window_attention(Q, K, V, T, "block") - full).max() < 1e-12
