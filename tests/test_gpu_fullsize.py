"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

The (batch, head) problems are independent, so the oracle checks sampled problems in full
(every chunk, every output row, every weight). The single 1M-token image-set chunk is too
long for the oracle inside a test; its sampled oracle values are stored in
tests/golden/imageset_oracle.npz by tests/golden/make_golden.py. Errors are max relative
errors |x - y|_inf / |y|_inf over the compared values."""
import os

import numpy as np
import pytest

import ttt_inputs as ti
from ttt_gpu import oracle_all, rel_err, run_gpu

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "imageset_oracle.npz")


def _compare(cfg, problems, tol):
    inp = ti.make_inputs(cfg)
    O, Ws = run_gpu(cfg, inp)
    ref = oracle_all(cfg, inp, problems)
    for p, (Or, Wr) in ref.items():
        eo = rel_err(O[p], Or)
        ew = [rel_err(Ws[m][p], Wr[m]) for m in range(len(Wr))]
        print(f"{cfg.name} problem {p}: O {eo:.3e} W {[f'{e:.3e}' for e in ew]}", flush=True)
        assert eo <= tol and max(ew) <= tol, (p, eo, ew)
        # renorm keeps every row at its initial norm
        if cfg.renorm:
            for m, w0 in enumerate(inp["w0"]):
                n0 = np.linalg.norm(w0[p[1]].astype(np.float64), axis=1)
                assert np.abs(np.linalg.norm(Ws[m][p], axis=1) / n0 - 1).max() < 1e-5


def test_lm_layer_full_size():
    _compare(ti.CONFIGS["lm"], [(0, 0), (3, 1)], 2e-2)


def test_long_context_full_size():
    _compare(ti.CONFIGS["long"], [(0, 1)], 2e-2)


def test_long_context_tiny_shape_full_size():
    _compare(ti.CONFIGS["long_alt"], [(0, 0)], 2e-2)


def test_small_chunk_full_size():
    _compare(ti.CONFIGS["smallchunk"], [(0, 0), (7, 11)], 2e-2)


def test_imageset_full_size():
    cfg = ti.CONFIGS["imageset"]
    g = np.load(GOLDEN)
    inp = ti.make_inputs(cfg)
    O, Ws = run_gpu(cfg, inp)
    eo = rel_err(O[0, 0][g["tokens"]], g["O"])
    ew = []
    for m in range(3):
        Wg = Ws[m][0, 0]
        ew.append(float(np.abs(Wg[g[f"W{m}_rows"]] - g[f"W{m}"]).max() / g[f"W{m}_absmax"]))
        assert np.abs(np.linalg.norm(Wg, axis=1) / g[f"W{m}_rownorm"] - 1).max() < 1e-5
    print(f"imageset: O {eo:.3e} W {[f'{e:.3e}' for e in ew]}", flush=True)
    assert eo <= 2e-2 and max(ew) <= 2e-2, (eo, ew)
