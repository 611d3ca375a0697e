"""Write the stored expected values for the full-size image-set workload.

The single 1,029,120-token chunk (128 views x 8040 patch tokens, dim 768, SwiGLU hidden
1536, Muon + row renorm, update then apply) takes the fp64 oracle minutes, too long for a
test, so its results are computed here once and stored: the final fast weights on a sample
of rows, their per-matrix max |value|, and the layer output on a sample of tokens.

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
N_ROWS = 24       # sampled rows per fast-weight matrix
N_TOKENS = 192    # sampled output tokens


def sample_indices(n, k, seed):
    return np.sort(np.random.default_rng(seed).choice(n, size=k, replace=False))


def main():
    cfg = ti.CONFIGS["imageset"]
    t = time.time()
    p = ti.make_problem_inputs(cfg, 0, 0)
    w0 = [w[0] for w in ti.make_weights(cfg)]
    print(f"inputs {time.time() - t:.1f} s", flush=True)
    tok = sample_indices(cfg.seq_len, N_TOKENS, 1)
    t = time.time()
    O, Ws = orc.sequence_forward(cfg, w0, p["q"], p["k"], p["v"], p["eta"], block_rows=8192,
                                 apply_rows=tok)
    print(f"oracle {time.time() - t:.1f} s", flush=True)
    out = {"tokens": tok, "O": O[tok]}
    for m, W in enumerate(Ws):
        rows = sample_indices(W.shape[0], N_ROWS, 10 + m)
        out[f"W{m}_rows"] = rows
        out[f"W{m}"] = W[rows]
        out[f"W{m}_absmax"] = np.abs(W).max()
        out[f"W{m}_rownorm"] = np.linalg.norm(W, axis=1)
    np.savez_compressed(OUT, **out)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
