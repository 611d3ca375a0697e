"""Plain fp64 CPU oracle of the LaCT block around the large-chunk TTT layer.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import or run this module. It shares no code with the HIP library.

[LaCT] "LaCT技术解析：大块测试时训练提升长序列建模效率" (peacm.com), §2.1 (Fig. 2): the block
stacks three kinds of layer -- window attention for the dependencies inside a chunk (a
sliding window for text, a window covering one whole image for image sets, §3.1), the
large-chunk TTT layer for the long-range ones, and a feed-forward layer for channel mixing.

Readings where the page is silent (each one is listed in the design notes):
* pre-norm residual sub-layers: h = x + attn(n(x)); h = h + ttt(n(h)); y = h + ffn(n(h)), with
  n the RMS normalisation without a learned scale, eps 1e-6;
* attention: heads of dim 128 over the model width, scores scaled by 1/sqrt(128), softmax
  over the window: "sliding" lets token t see tokens t-window+1 .. t, "block" lets it see
  every token of its own block of `window` tokens (an image); one projection [3D x D] to
  q, k, v and one [D x D] back;
* TTT sub-layer: q, k, v = n(h) W^T split into the TTT heads (heads x dim = D), q and k
  L2-normalised per head and token (the layer's stated input distribution), eta = 0.01
  sigmoid(n(h) . w_eta[head]); the layer's inputs and outputs are in its activation dtype
  (bf16 values: the oracle rounds them as the layer's interface does), then an output
  projection [D x D];
* feed-forward: the standard Transformer MLP, W2 gelu(W1 x) with hidden 4D and the exact
  erf GELU, no biases.
* storage: the block runs in bf16 with fp32 accumulation, so every activation a sub-layer
  hands on (the normalised rows, the projections, the attention and TTT outputs, the MLP
  hidden, the residual stream) is a bf16 value; the oracle rounds there and computes
  everything between those points in fp64.
Weights are given as bf16 values (the model's dtype), inputs as bf16 values.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

import oracle.ttt_oracle as orc

EPS = 1e-6
ATTN_HEAD_DIM = 128


def bf16(x):
    """Round to bfloat16 (nearest even) and back, as the layer's interface stores values."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (((u + bias) >> np.uint32(16)) << np.uint32(16)).view(np.float32).astype(np.float64)


def rmsnorm(x):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + EPS)


def gelu(z):
    return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


def window_mask(T: int, window: int, mode: str) -> np.ndarray:
    """allowed[t, j]: may token t attend to token j."""
    t = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    if mode == "sliding":
        return (j <= t) & (j > t - window)
    if mode == "block":
        return (j // window) == (t // window)
    raise ValueError(mode)


def window_attention(Q, K, V, window: int, mode: str):
    """softmax(Q K^T / sqrt(d) restricted to the window) V for one head, Q/K/V [T, d]."""
    Q, K, V = (np.asarray(a, np.float64) for a in (Q, K, V))
    S = Q @ K.T / np.sqrt(Q.shape[1])
    S = np.where(window_mask(len(Q), window, mode), S, -np.inf)
    S = S - S.max(axis=1, keepdims=True)
    P = np.exp(S)
    return (P / P.sum(axis=1, keepdims=True)) @ V


def attention_layer(X, w_qkv, w_out, window: int, mode: str):
    """Multi-head window attention over rows of X [T, D] ([LaCT] §2.1 window attention):
    returns (the heads' outputs before the output projection, the projected output), both
    as the stored bf16 values."""
    D = X.shape[1]
    qkv = bf16(X @ np.asarray(w_qkv, np.float64).T)
    heads = D // ATTN_HEAD_DIM
    out = np.zeros_like(X)
    for h in range(heads):
        s = slice(h * ATTN_HEAD_DIM, (h + 1) * ATTN_HEAD_DIM)
        out[:, s] = window_attention(qkv[:, s], qkv[:, D:][:, s], qkv[:, 2 * D:][:, s],
                                     window, mode)
    out = bf16(out)
    return out, out @ np.asarray(w_out, np.float64).T


def ttt_inputs(X, w_qkv, w_eta, heads: int, dim: int):
    """The TTT sub-layer's inputs from its normalised rows X [T, D]: per head q and k
    L2-normalised, v, all bf16 values, and eta fp32 values. Returns lists per head."""
    D = X.shape[1]
    qkv = bf16(X @ np.asarray(w_qkv, np.float64).T)
    eta = 0.01 / (1.0 + np.exp(-(X @ np.asarray(w_eta, np.float64).T)))   # [T, H]
    out = []
    for h in range(heads):
        q = qkv[:, h * dim:(h + 1) * dim]
        k = qkv[:, D + h * dim:D + (h + 1) * dim]
        v = qkv[:, 2 * D + h * dim:2 * D + (h + 1) * dim]
        out.append((bf16(q / np.linalg.norm(q, axis=1, keepdims=True)),
                    bf16(k / np.linalg.norm(k, axis=1, keepdims=True)), v,
                    eta[:, h].astype(np.float32).astype(np.float64)))
    return out


def ttt_layer(X, w_qkv, w_eta, w_out, tcfg, W0s_per_head):
    """The TTT sub-layer on rows of X [T, D]: ttt_inputs, the oracle's sequence_forward per
    head ([LaCT] §2.1 large-chunk TTT layer), output projection. Returns (the layer's bf16
    outputs [T, H d], the projected output, each head's state at the end)."""
    H, d = tcfg.heads, tcfg.dim
    O = np.zeros((len(X), H * d))
    states = []
    for h, (q, k, v, e) in enumerate(ttt_inputs(X, w_qkv, w_eta, H, d)):
        Oh, Wh = orc.sequence_forward(tcfg, W0s_per_head[h], q, k, v, e)
        O[:, h * d:(h + 1) * d] = bf16(Oh)
        states.append(Wh)
    return O, O @ np.asarray(w_out, np.float64).T, states


def ffn_layer(X, w_up, w_down):
    """The standard Transformer MLP ([LaCT] §2.1 feed-forward layer), bf16 hidden."""
    return bf16(gelu(X @ np.asarray(w_up, np.float64).T)) @ np.asarray(w_down, np.float64).T


def block_forward(bcfg, weights, X, W0s_per_head, return_states: bool = False):
    """One block for one sequence X [T, D] (bf16 values): returns y [T, D] (bf16 values),
    and with return_states also the TTT heads' states at the sequence's end."""
    X = np.asarray(X, np.float64)
    _, a = attention_layer(bf16(rmsnorm(X)), weights["attn_qkv"], weights["attn_out"],
                           bcfg.window, bcfg.window_mode)
    h = bf16(X + a)
    _, t, states = ttt_layer(bf16(rmsnorm(h)), weights["ttt_qkv"], weights["ttt_eta"],
                             weights["ttt_out"], bcfg.ttt, W0s_per_head)
    h = bf16(h + t)
    y = bf16(h + ffn_layer(bf16(rmsnorm(h)), weights["ffn_up"], weights["ffn_down"]))
    return (y, states) if return_states else y
