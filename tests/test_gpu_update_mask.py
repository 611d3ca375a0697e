"""Chunks that do not update the fast weights (ttt_sequence_forward_masked): GPU against
the oracle with the same flags, and bitwise against the unmasked call (all flags set) and
against eta zeroed on the skipped chunks (no weight decay).  The LaCT page (§3.3) updates
the fast weights of its video model on clean-frame chunks only; alternate flags stand in
for that sequence, and flags at a stride with the update-then-apply order for updates on
every s-th chunk."""
import numpy as np
import pytest
import torch

import oracle.ttt_oracle as orc
import ttt_inputs as ti
import weight_sequence_layers_amd as W
from ttt_gpu import device_inputs, read_state, rel_err

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _run(cfg, inp, mask, planes=None, path="auto", eta=None):
    c = W.make_config(cfg, planes=planes, path=path)
    q, k, v, e, w0 = device_inputs(cfg, inp)
    if eta is not None:
        e = torch.from_numpy(np.ascontiguousarray(eta)).cuda()
    out = torch.empty_like(q)
    st = W.ttt_init_state(c, w0)
    if mask is None:
        W.ttt_sequence_forward(st, q, k, v, e, out, cfg.seq_len)
    else:
        W.ttt_sequence_forward_masked(st, q, k, v, e, out, cfg.seq_len, mask)
    Ws, _ = read_state(c, st)
    W.ttt_state_health(st)
    O = out.float().cpu().numpy()
    raw = out.view(torch.int16).cpu().numpy() if cfg.act == "bf16" else O
    st.destroy()
    return O, Ws, raw


CASES = {
    "swiglu_muon_bf16_alternate": (ti.Config("mask_a", 2, 2, 1536, 256, 128, 256, "swiglu",
                                             "dot", 5, True, "bf16", "apply_then_update", 81),
                                   (0, 1, 0, 1, 0, 1)),
    "swiglu_muon_bf16_stride3_update_first": (ti.Config("mask_b", 1, 2, 1536, 256, 128, 256,
                                                        "swiglu", "dot", 5, True, "bf16",
                                                        "update_then_apply", 82),
                                              (1, 0, 0, 1, 0, 0)),
    "gelu_mse_f32": (ti.Config("mask_c", 2, 1, 900, 300, 80, 176, "gelu", "mse", 0, False,
                               "f32", "apply_then_update", 83), (1, 0, 1)),
    "linear_dot_f32_decay": (ti.Config("mask_d", 1, 2, 800, 200, 64, 64, "linear", "dot", 0,
                                       False, "f32", "apply_then_update", 84, lr=(0.5,),
                                       weight_decay=0.1), (0, 1, 1, 0)),
    "resident_small_chunk": (ti.Config("mask_e", 2, 3, 640, 64, 64, 256, "gelu", "mse", 0,
                                       False, "bf16", "apply_then_update", 85),
                             (1, 1, 0, 0, 1, 0, 1, 1, 1, 0)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_masked_parity(name):
    cfg, mask = CASES[name]
    inp = ti.make_inputs(cfg)
    planes = (1, 1, 1, 0) if name.startswith("resident") else None
    O, Ws, _ = _run(cfg, inp, mask, planes)
    ref = orc.forward_all(cfg, inp, update_chunks=mask)
    tol = TOL[cfg.act]
    for (b, h), (Or, Wr) in ref.items():
        eo = rel_err(O[b, h], Or)
        ew = [rel_err(Ws[m][b, h], Wr[m]) for m in range(len(Wr))]
        print(f"{name} problem ({b},{h}): O {eo:.3e} W {[f'{e:.3e}' for e in ew]}", flush=True)
        assert eo <= tol and max(ew) <= tol, (b, h, eo, ew)


@pytest.mark.parametrize("path", ["staged", "resident"])
def test_all_flags_equal_the_unmasked_call(path):
    if path == "staged":
        cfg = ti.Config("mask_f", 1, 2, 1024, 256, 64, 128, "swiglu", "dot", 5, True, "bf16",
                        "apply_then_update", 86)
        planes = None
    else:
        cfg, planes = CASES["resident_small_chunk"][0], (1, 1, 1, 0)
    inp = ti.make_inputs(cfg)
    _, W1, r1 = _run(cfg, inp, [1] * cfg.n_chunks, planes, path)
    _, W2, r2 = _run(cfg, inp, None, planes, path)
    assert np.array_equal(r1, r2)
    assert all(np.array_equal(a, b) for a, b in zip(W1, W2))


@pytest.mark.parametrize("path", ["staged", "resident"])
def test_skipped_chunk_equals_zero_eta(path):
    # with no decay a chunk that does not update leaves the state as eta = 0 does; on the
    # staged path the outputs agree bitwise too (the resident loop answers its own chunks
    # with its own rounding, so there only the state is compared bitwise)
    if path == "staged":
        cfg = ti.Config("mask_g", 2, 1, 1024, 256, 64, 128, "swiglu", "dot", 5, True, "bf16",
                        "apply_then_update", 87)
        planes, mask = None, (1, 0, 1, 0)
    else:
        cfg, mask = CASES["resident_small_chunk"]
        planes = (1, 1, 1, 0)
    inp = ti.make_inputs(cfg)
    eta0 = inp["eta"].copy()
    for c, m in enumerate(mask):
        if not m:
            eta0[:, :, c * cfg.chunk:(c + 1) * cfg.chunk] = 0.0
    O1, W1, r1 = _run(cfg, inp, mask, planes, path)
    O2, W2, r2 = _run(cfg, inp, None, planes, path, eta=eta0)
    assert all(np.array_equal(a, b) for a, b in zip(W1, W2))
    if path == "staged":
        assert np.array_equal(r1, r2)
    else:
        assert rel_err(O1, O2) < 1e-2


def test_wrong_flag_count_is_refused():
    cfg = ti.Config("mask_h", 1, 1, 512, 256, 64, 128, "swiglu", "dot", 0, True, "bf16",
                    "apply_then_update", 88)
    inp = ti.make_inputs(cfg)
    c = W.make_config(cfg)
    q, k, v, e, w0 = device_inputs(cfg, inp)
    st = W.ttt_init_state(c, w0)
    with pytest.raises(ValueError):
        W.ttt_sequence_forward_masked(st, q, k, v, e, torch.empty_like(q), cfg.seq_len, [1])
    st.destroy()
