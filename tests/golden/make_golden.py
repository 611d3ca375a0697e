"""Write the stored expected values for the full-size image-set workload.

The single 1,029,120-token chunk (128 views x 8040 patch tokens, dim 768, SwiGLU hidden
1536, Muon + row renorm, update then apply) takes the fp64 oracle minutes, too long for a
test, so its results are computed here once and stored:

* for every matrix, two whole rows from every 128-row tile of it (each whole row spans
  every column tile, so every 128 x 128 tile of the matrix, and of its transpose, holds
  stored values), the matrix's max |value| and every row's L2 norm;
* the layer output at the first and last token of every 65536-token block of the sequence
  and at 16 more tokens of each block, each from a different 128-token tile of it.

Only the oracle and the seeded input generator are called.

    python tests/golden/make_golden.py     # writes tests/golden/imageset_oracle.npz
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle.ttt_oracle as orc  # noqa: E402
import ttt_inputs as ti  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "imageset_oracle.npz")
TILE = 128            # row tile of the GPU kernels
ROWS_PER_TILE = 2     # stored rows per row tile of each matrix
BLOCK = 65536         # tokens per apply launch
TOKENS_PER_BLOCK = 16 # stored tokens per block besides its first and last


def tile_rows(n, seed):
    """ROWS_PER_TILE distinct rows from every TILE-row tile of an n-row matrix."""
    rng = np.random.default_rng(seed)
    rows = []
    for t0 in range(0, n, TILE):
        rows.extend(t0 + rng.choice(min(TILE, n - t0), size=ROWS_PER_TILE, replace=False))
    return np.sort(np.array(rows))


def block_tokens(T, seed):
    """First and last token of every BLOCK-token block, plus TOKENS_PER_BLOCK tokens of it
    from distinct TILE-token tiles."""
    rng = np.random.default_rng(seed)
    toks = []
    for b0 in range(0, T, BLOCK):
        n = min(BLOCK, T - b0)
        tiles = rng.choice((n + TILE - 1) // TILE, size=TOKENS_PER_BLOCK, replace=False)
        for t in tiles:
            toks.append(b0 + t * TILE + rng.integers(min(TILE, n - t * TILE)))
        toks += [b0, b0 + n - 1]
    return np.unique(np.array(toks))


def main():
    cfg = ti.CONFIGS["imageset"]
    t = time.time()
    p = ti.make_problem_inputs(cfg, 0, 0)
    w0 = [w[0] for w in ti.make_weights(cfg)]
    print(f"inputs {time.time() - t:.1f} s", flush=True)
    tok = block_tokens(cfg.seq_len, 1)
    t = time.time()
    O, Ws = orc.sequence_forward(cfg, w0, p["q"], p["k"], p["v"], p["eta"], block_rows=8192,
                                 apply_rows=tok)
    print(f"oracle {time.time() - t:.1f} s", flush=True)
    out = {"tokens": tok, "O": O[tok]}
    for m, W in enumerate(Ws):
        rows = tile_rows(W.shape[0], 10 + m)
        out[f"W{m}_rows"] = rows
        out[f"W{m}"] = W[rows]
        out[f"W{m}_absmax"] = np.abs(W).max()
        out[f"W{m}_rownorm"] = np.linalg.norm(W, axis=1)
    np.savez_compressed(OUT, **out)
    print("wrote", OUT, {k: v.shape for k, v in out.items()})


if __name__ == "__main__":
    main()
