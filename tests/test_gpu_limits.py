"""GPU parity at the library's size limits: the largest dim and hidden (1024, 4096) under
Muon and renorm, the largest problem count (batch x heads = 65535) on tiny matrices, and
dims that are multiples of 16 but not of the 64-wide tiles. Errors are max relative errors
|x - y|_inf / |y|_inf against the oracle; 1e-4 for fp32 activations (three planes), 2e-2
for bf16 activations."""
import numpy as np
import pytest

import ttt_inputs as ti
from ttt_gpu import oracle_all, parity, rel_err, run_gpu

pytestmark = pytest.mark.gpu


def test_largest_dim_and_hidden():
    cfg = ti.Config("maxdim", 1, 1, 256, 128, 1024, 4096, "swiglu", "dot", 5, True, "bf16",
                    "apply_then_update", 77)
    inp = ti.make_inputs(cfg)
    O, Ws = run_gpu(cfg, inp)
    eo, ew = parity(cfg, inp, O, Ws)
    print(f"dim 1024 hidden 4096: O {eo:.3e} W {[f'{e:.3e}' for e in ew]}", flush=True)
    assert eo <= 2e-2 and max(ew) <= 2e-2, (eo, ew)


def test_most_problems():
    # batch * heads = 65535 (the limit), tiny matrices; sampled problems against the oracle
    cfg = ti.Config("maxprob", 4369, 15, 32, 16, 16, 32, "swiglu", "dot", 5, True, "f32",
                    "apply_then_update", 78)
    inp = ti.make_inputs(cfg)
    O, Ws = run_gpu(cfg, inp)
    probs = [(0, 0), (1234, 7), (4368, 14)]
    ref = oracle_all(cfg, inp, probs)
    for p, (Or, Wr) in ref.items():
        eo = rel_err(O[p], Or)
        ew = max(rel_err(Ws[m][p], Wr[m]) for m in range(3))
        print(f"problem {p}: O {eo:.3e} W {ew:.3e}", flush=True)
        assert eo <= 1e-4 and ew <= 1e-4, (p, eo, ew)


@pytest.mark.parametrize("dim,hidden", [(16, 16), (48, 208), (1008, 2032)])
def test_dims_off_the_tile_grid(dim, hidden):
    cfg = ti.Config("odd", 1, 2, 96, 48, dim, hidden, "swiglu", "dot", 5, True, "f32",
                    "apply_then_update", 79)
    inp = ti.make_inputs(cfg)
    O, Ws = run_gpu(cfg, inp)
    eo, ew = parity(cfg, inp, O, Ws)
    print(f"dim {dim} hidden {hidden}: O {eo:.3e} W {[f'{e:.3e}' for e in ew]}", flush=True)
    assert eo <= 1e-4 and max(ew) <= 1e-4, (eo, ew)
