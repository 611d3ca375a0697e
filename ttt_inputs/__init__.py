"""Seeded synthetic inputs and the workload registry for the large-chunk TTT layer.

This module is the one piece shared by the CPU oracle and the HIP path. It holds
no arithmetic of the method itself: it only draws random numbers, normalises
query/key vectors (an input-distribution choice) and rounds values to the
activation dtype.

Every tensor is generated in blocks of ``TOKEN_BLOCK`` tokens, each block from
its own counter-keyed numpy ``SeedSequence`` (entropy = seed, spawn key =
(tensor id, batch, head, block)). Any (batch, head) problem, or any token block
of it, can therefore be regenerated on its own and is bit-identical to the
same slice of the whole tensor.

Distributions (the workloads' stated inputs):
  * fast-weight init W ~ N(0, 1/d) per head, fp32, shared across the batch;
  * q, k ~ N(0, 1), each token vector L2-normalised (in fp64), then stored in
    the activation dtype with round-to-nearest-even;
  * v ~ N(0, 1), stored in the activation dtype;
  * eta_t = 0.01 * sigmoid(N(0, 1)), fp32.
For the block around the layer (make_block_inputs):
  * the block input x ~ N(0, 1) per token and channel, bf16;
  * every projection weight [out][in] ~ N(0, 1 / in), bf16 (the usual fan-in scaling, so
    each projection keeps the scale of its input).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

TOKEN_BLOCK = 65536

# tensor ids used as the first spawn-key element
_TID = {"W1": 0, "W3": 1, "W2": 2, "q": 3, "k": 4, "v": 5, "eta": 6, "W": 7,
        "x": 8, "attn_qkv": 9, "attn_out": 10, "ttt_qkv": 11, "ttt_eta": 12, "ttt_out": 13,
        "ffn_up": 14, "ffn_down": 15}


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    batch: int
    heads: int
    seq_len: int
    chunk: int
    dim: int            # d, the head dimension
    hidden: int         # dh, fast-weight hidden width (ignored for 'linear')
    fw: str = "swiglu"  # 'swiglu' | 'gelu' | 'linear'
    loss: str = "dot"   # 'dot' (-sum eta <f(k),v>) | 'mse' (sum eta ||f(k)-v||^2)
    ns_steps: int = 0   # 0: plain gradient step; 5: Newton-Schulz orthogonalised step
    renorm: bool = False
    act: str = "f32"    # 'f32' | 'bf16'
    order: str = "apply_then_update"  # | 'update_then_apply'
    seed: int = 1000
    lr: Tuple[float, ...] = ()   # step size per matrix (state order); () or 0 entries: 1
    weight_decay: float = 0.0    # decay of the state per chunk, in [0, 1)
    momentum: float = 0.0        # heavy-ball coefficient over chunk gradients, in [0, 1)

    def step_sizes(self) -> List[float]:
        """The step size of each matrix, defaults filled in."""
        n = len(self.matrix_names())
        lr = list(self.lr) + [0.0] * (n - len(self.lr))
        return [x if x != 0 else 1.0 for x in lr[:n]]

    @property
    def n_chunks(self) -> int:
        return 0 if self.seq_len == 0 else self.seq_len // self.chunk

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    def matrix_names(self) -> List[str]:
        return {"swiglu": ["W1", "W3", "W2"], "gelu": ["W1", "W2"], "linear": ["W"]}[self.fw]

    def matrix_shapes(self) -> List[tuple]:
        d, dh = self.dim, self.hidden
        return {"swiglu": [(dh, d), (dh, d), (d, dh)],
                "gelu": [(dh, d), (d, dh)],
                "linear": [(d, d)]}[self.fw]


# The five workloads. Index 0 is the tiny fp32 case, 1 the chunk-2048 language-model
# layer (the headline), 2 the 128K long-context variant at the LM layer shape
# (2-alt: the same at the tiny shape), 3 the single 1,029,120-token image-set chunk,
# 4 the classic small-chunk MLP/MSE case.
CONFIGS: Dict[str, Config] = {
    "tiny": Config("tiny", 1, 1, 2048, 512, 64, 128, "swiglu", "dot", 0, True, "f32",
                   "apply_then_update", 1001),
    "lm": Config("lm", 4, 2, 32768, 2048, 512, 1024, "swiglu", "dot", 5, True, "bf16",
                 "apply_then_update", 1002),
    "long": Config("long", 1, 2, 131072, 4096, 512, 1024, "swiglu", "dot", 5, True, "bf16",
                   "apply_then_update", 1003),
    "long_alt": Config("long_alt", 1, 1, 131072, 4096, 64, 128, "swiglu", "dot", 5, True,
                       "bf16", "apply_then_update", 1003),
    "imageset": Config("imageset", 1, 1, 1029120, 1029120, 768, 1536, "swiglu", "dot", 5,
                       True, "bf16", "update_then_apply", 1004),
    "smallchunk": Config("smallchunk", 8, 12, 32768, 64, 64, 256, "gelu", "mse", 0, False,
                         "bf16", "apply_then_update", 1005),
}


def bf16_round(x: np.ndarray):
    """Round fp32 values to bfloat16 (round-to-nearest-even).

    Returns (values as float32 holding exact bf16 numbers, raw uint16 bits)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    bits = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    vals = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return vals, bits


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=tuple(key)))


def make_weights(cfg: Config, seed: Optional[int] = None) -> List[np.ndarray]:
    """Initial fast weights per head, fp32, list of arrays shaped [H, rows, cols]."""
    seed = cfg.seed if seed is None else seed
    out = []
    for name, shape in zip(cfg.matrix_names(), cfg.matrix_shapes()):
        per_head = []
        for h in range(cfg.heads):
            g = _rng(seed, _TID[name], h).standard_normal(shape)
            per_head.append((g / np.sqrt(cfg.dim)).astype(np.float32))
        out.append(np.stack(per_head))
    return out


def _token_block(cfg: Config, seed: int, name: str, b: int, h: int, blk: int, n: int):
    rng = _rng(seed, _TID[name], b, h, blk)
    if name == "eta":
        z = rng.standard_normal(n)
        return (0.01 / (1.0 + np.exp(-z))).astype(np.float32)
    x = rng.standard_normal((n, cfg.dim), dtype=np.float32)
    if name in ("q", "k"):
        x64 = x.astype(np.float64)
        x = (x64 / np.linalg.norm(x64, axis=1, keepdims=True)).astype(np.float32)
    return x


def make_problem_inputs(cfg: Config, b: int, h: int, seed: Optional[int] = None,
                        t0: int = 0, t1: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Inputs of one (batch, head) problem for tokens [t0, t1).

    q, k, v come back as float32 arrays [n, d] holding exactly the act-dtype values
    the device receives; for bf16 also 'q_bits' etc. (uint16). eta is float32 [n]."""
    seed = cfg.seed if seed is None else seed
    t1 = cfg.seq_len if t1 is None else t1
    out: Dict[str, np.ndarray] = {}
    for name in ("q", "k", "v", "eta"):
        parts = []
        for blk in range(t0 // TOKEN_BLOCK, (max(t1, 1) - 1) // TOKEN_BLOCK + 1):
            lo = blk * TOKEN_BLOCK
            n = min(TOKEN_BLOCK, cfg.seq_len - lo)
            if n <= 0:
                break
            x = _token_block(cfg, seed, name, b, h, blk, n)
            parts.append(x[max(t0 - lo, 0):max(min(t1 - lo, n), 0)])
        shape = (0,) if name == "eta" else (0, cfg.dim)
        x = np.concatenate(parts) if parts else np.zeros(shape, np.float32)
        if name != "eta" and cfg.act == "bf16":
            x, bits = bf16_round(x)
            out[name + "_bits"] = bits
        out[name] = x
    return out


def make_inputs(cfg: Config, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """All inputs: 'w0' (list of [H, ...] fp32), q/k/v [B, H, T, d] (float32 values of
    the act dtype; plus uint16 '*_bits' for bf16) and eta [B, H, T] float32."""
    seed = cfg.seed if seed is None else seed
    B, H, T, d = cfg.batch, cfg.heads, cfg.seq_len, cfg.dim
    res: Dict[str, np.ndarray] = {"w0": make_weights(cfg, seed)}
    res["q"] = np.empty((B, H, T, d), np.float32)
    res["k"] = np.empty((B, H, T, d), np.float32)
    res["v"] = np.empty((B, H, T, d), np.float32)
    res["eta"] = np.empty((B, H, T), np.float32)
    if cfg.act == "bf16":
        for n in ("q", "k", "v"):
            res[n + "_bits"] = np.empty((B, H, T, d), np.uint16)
    for b in range(B):
        for h in range(H):
            p = make_problem_inputs(cfg, b, h, seed)
            for key, val in p.items():
                res[key][b, h] = val
    return res


BLOCK_WEIGHT_NAMES = ("attn_qkv", "attn_out", "ttt_qkv", "ttt_eta", "ttt_out", "ffn_up",
                      "ffn_down")


def block_weight_shapes(dim: int, ffn_hidden: int, ttt_heads: int) -> Dict[str, tuple]:
    D, F = dim, ffn_hidden
    return {"attn_qkv": (3 * D, D), "attn_out": (D, D), "ttt_qkv": (3 * D, D),
            "ttt_eta": (ttt_heads, D), "ttt_out": (D, D), "ffn_up": (F, D), "ffn_down": (D, F)}


def make_block_inputs(batch: int, seq_len: int, dim: int, ffn_hidden: int, ttt_heads: int,
                      seed: int) -> Dict[str, np.ndarray]:
    """The block's input x [batch, seq_len, dim] and its projection weights, as float32
    arrays of bf16 values (plus '<name>_bits' uint16). x is drawn per (batch, token block),
    so any batch element or token block regenerates on its own."""
    out: Dict[str, np.ndarray] = {}
    for name, (o, i) in block_weight_shapes(dim, ffn_hidden, ttt_heads).items():
        w = _rng(seed, _TID[name]).standard_normal((o, i), dtype=np.float32) / np.float32(np.sqrt(i))
        out[name], out[name + "_bits"] = bf16_round(w)
    x = np.empty((batch, seq_len, dim), np.float32)
    for b in range(batch):
        for blk in range((seq_len + TOKEN_BLOCK - 1) // TOKEN_BLOCK):
            lo = blk * TOKEN_BLOCK
            n = min(TOKEN_BLOCK, seq_len - lo)
            x[b, lo:lo + n] = _rng(seed, _TID["x"], b, blk).standard_normal((n, dim),
                                                                            dtype=np.float32)
    out["x"], out["x_bits"] = bf16_round(x)
    return out
