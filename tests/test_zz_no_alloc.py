"""The allocation-free sequence call (ttt_sequence_forward_noalloc) against the existing
entry point: the same configuration, weights and inputs through ttt_init_state +
ttt_sequence_forward must give the same outputs and final state, bit for bit (the two run
the same kernels on the same launch grid; only where the workspace lives differs).  Two
calls in a row on the shared per-GPU workspace, the second with a smaller input, so that
leftovers of the first call cannot go unseen.  Runs last: its workspace array stays
allocated on the GPU for the rest of the process."""
import numpy as np
import pytest
import torch

import ttt_inputs as ti
import weight_sequence_layers_amd as W
from ttt_gpu import device_inputs

pytestmark = pytest.mark.gpu


def _reference(cfg, inp, planes):
    c = W.make_config(cfg, planes=planes)
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    out = torch.empty_like(q)
    st = W.ttt_init_state(c, w0)
    W.ttt_sequence_forward(st, q, k, v, eta, out, cfg.seq_len)
    flat = torch.empty(W.ttt_state_numel(c), dtype=torch.float32, device="cuda")
    W.ttt_get_state(st, flat)
    torch.cuda.synchronize()
    st.destroy()
    return out, flat


def _noalloc(cfg, inp, planes):
    c = W.make_config(cfg, planes=planes)
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    # the state buffer starts as every batch element's copy of its head's initial weights
    state = torch.cat([w.reshape(1, cfg.heads, -1).expand(cfg.batch, -1, -1).reshape(-1)
                       for w in torch.split(w0, [cfg.heads * r * cc for r, cc in
                                                cfg.matrix_shapes()])]).contiguous()
    out = torch.full_like(q, float("nan"))
    W.ttt_sequence_forward_noalloc(c, state, q, k, v, eta, out, cfg.seq_len)
    torch.cuda.synchronize()
    return out, state


CASES = [
    # a larger call, then a smaller one (fewer problems, shorter sequence, smaller dims)
    (ti.Config("na_big", 2, 3, 2048, 512, 128, 256, "swiglu", "dot", 5, True, "bf16",
               "apply_then_update", 71), (1, 2, 2, 0)),
    (ti.Config("na_small", 1, 1, 512, 128, 64, 128, "swiglu", "dot", 5, True, "bf16",
               "apply_then_update", 72), (1, 2, 2, 0)),
]


def test_noalloc_matches_the_state_entry_point_on_two_calls():
    for cfg, planes in CASES:
        print(f"noalloc case {cfg.name}: B={cfg.batch} H={cfg.heads} T={cfg.seq_len} "
              f"d={cfg.dim} dh={cfg.hidden}", flush=True)
        inp = ti.make_inputs(cfg)
        o_ref, w_ref = _reference(cfg, inp, planes)
        o, w = _noalloc(cfg, inp, planes)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), cfg.name
        assert torch.equal(w, w_ref), cfg.name


def test_noalloc_small_chunk_resident_and_fp32_staged():
    """The resident small-chunk loop (its state updated in place in the caller's buffer)
    and an fp32 configuration on the staged path, each after the calls above."""
    cases = [
        (ti.Config("na_res", 2, 2, 1024, 64, 64, 256, "gelu", "mse", 0, False, "bf16",
                   "apply_then_update", 73), (1, 1, 1, 0)),
        (ti.Config("na_f32", 1, 2, 1024, 256, 64, 128, "swiglu", "dot", 0, True, "f32",
                   "apply_then_update", 74), (3, 3, 3, 0)),
    ]
    for cfg, planes in cases:
        print(f"noalloc case {cfg.name}", flush=True)
        inp = ti.make_inputs(cfg)
        o_ref, w_ref = _reference(cfg, inp, planes)
        o, w = _noalloc(cfg, inp, planes)
        assert torch.equal(o.view(torch.int16) if cfg.act == "bf16" else o,
                           o_ref.view(torch.int16) if cfg.act == "bf16" else o_ref), cfg.name
        assert torch.equal(w, w_ref), cfg.name


def test_noalloc_rejects_an_oversized_configuration():
    cfg = ti.CONFIGS["lm"]
    c = W.make_config(cfg)
    x = torch.zeros(16, device="cuda")
    with pytest.raises(W.TTTError) as e:
        W.ttt_sequence_forward_noalloc(c, x, x, x, x, x, x, cfg.chunk)
    assert e.value.status == 2 and "workspace" in str(e.value)
