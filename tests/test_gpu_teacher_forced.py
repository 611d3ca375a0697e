"""Teacher-forced per-chunk parity on the GPU at the Muon workloads' layer shapes.

Under Muon the state trajectory amplifies any rounding by about 1.28x per chunk, so the
end-to-end comparisons elsewhere measure kernel error times that growth. Here the oracle
takes one chunk step from the state the GPU itself holds before the chunk, and the GPU's
outputs and state after that chunk are compared with it: this is the error of one step
of the kernels, with no trajectory behind it. Errors are max relative errors
|x - y|_inf / |y|_inf per tensor; the per-step bound asserted for the state is ten times
below the end-to-end bound."""
import numpy as np
import pytest
import torch

import oracle.ttt_oracle as orc
import ttt_inputs as ti
import weight_sequence_layers_amd as W
from ttt_gpu import device_inputs, read_state, rel_err

pytestmark = pytest.mark.gpu

STATE_TOL = 2e-3   # one step of the state path
OUT_TOL = 2e-2     # outputs: the apply path runs on one bf16 plane


def _teacher_forced(cfg, checks):
    c = W.make_config(cfg)
    inp = ti.make_inputs(cfg)
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    st = W.ttt_init_state(c, w0)
    b = cfg.chunk
    worst_o, worst_w = 0.0, 0.0
    for ci in range(max(checks) + 1):
        sl = slice(ci * b, (ci + 1) * b)
        prev = read_state(c, st)[0] if ci in checks else None
        oc = torch.empty_like(q[:, :, sl].contiguous())
        W.ttt_chunk_forward(st, q[:, :, sl].contiguous(), k[:, :, sl].contiguous(),
                            v[:, :, sl].contiguous(), eta[:, :, sl].contiguous(), oc)
        if ci not in checks:
            continue
        after = read_state(c, st)[0]
        O = oc.float().cpu().numpy()
        for bb in range(cfg.batch):
            for h in range(cfg.heads):
                W_prev = [m[bb, h] for m in prev]
                O_ref, W_ref = orc.sequence_forward(
                    cfg.replace(seq_len=b), W_prev, inp["q"][bb, h, sl], inp["k"][bb, h, sl],
                    inp["v"][bb, h, sl], inp["eta"][bb, h, sl])
                eo = rel_err(O[bb, h], O_ref)
                ew = max(rel_err(after[m][bb, h], W_ref[m]) for m in range(len(W_ref)))
                print(f"{cfg.name} chunk {ci} problem ({bb},{h}): O {eo:.2e} W {ew:.2e}",
                      flush=True)
                worst_o, worst_w = max(worst_o, eo), max(worst_w, ew)
    W.ttt_state_health(st)
    st.destroy()
    assert worst_o <= OUT_TOL and worst_w <= STATE_TOL, (worst_o, worst_w)


def test_lm_shape_one_step_at_a_time():
    # the LM layer (dim 512, hidden 1024, chunk 2048, Muon, renorm), one batch element
    _teacher_forced(ti.CONFIGS["lm"].replace(batch=1), checks=[0, 5, 15])


def test_long_context_shape_one_step_at_a_time():
    # chunk 4096 with the long-context precision preset
    _teacher_forced(ti.CONFIGS["long"].replace(heads=1, seq_len=4096 * 12), checks=[0, 11])
