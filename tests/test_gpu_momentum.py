"""Heavy-ball momentum over chunks (ttt_config.momentum): GPU against the oracle, the
state holding the fast weights followed by the momentum buffers; resume through
ttt_get_state / ttt_set_state carries the buffers (bitwise against an uninterrupted run);
chunks without update leave the buffers alone."""
import numpy as np
import pytest
import torch

import oracle.ttt_oracle as orc
import ttt_inputs as ti
import weight_sequence_layers_amd as W
from ttt_gpu import device_inputs, parity, read_state, run_gpu

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}

CASES = {
    "swiglu_muon_bf16": ti.Config("mo_a", 2, 2, 1024, 256, 128, 256, "swiglu", "dot", 5, True,
                                  "bf16", "apply_then_update", 111, momentum=0.9),
    "swiglu_muon_f32_step": ti.Config("mo_b", 1, 2, 768, 256, 80, 176, "swiglu", "dot", 5,
                                      True, "f32", "update_then_apply", 112, lr=(0.5, 1.2, 0.8),
                                      weight_decay=0.05, momentum=0.5),
    "gelu_mse_f32": ti.Config("mo_c", 2, 1, 600, 200, 64, 256, "gelu", "mse", 0, False, "f32",
                              "apply_then_update", 113, momentum=0.8),
    "linear_dot_f32": ti.Config("mo_d", 1, 2, 512, 128, 64, 64, "linear", "dot", 0, False,
                                "f32", "apply_then_update", 114, momentum=0.6),
    "token_split_bf16": ti.Config("mo_e", 1, 2, 2000, 1000, 64, 128, "swiglu", "dot", 5, True,
                                  "bf16", "apply_then_update", 115, momentum=0.7),
}


@pytest.mark.parametrize("name", list(CASES))
def test_momentum_parity(name):
    cfg = CASES[name]
    inp = ti.make_inputs(cfg)
    O, Ws = run_gpu(cfg, inp)
    assert len(Ws) == 2 * len(cfg.matrix_shapes())
    eo, ew = parity(cfg, inp, O, Ws)
    print(f"{name}: O {eo:.3e} W+M {[f'{e:.3e}' for e in ew]}", flush=True)
    tol = TOL[cfg.act]
    assert eo <= tol and max(ew) <= tol, (eo, ew)


def test_momentum_resume_through_get_and_set_state():
    cfg = CASES["swiglu_muon_bf16"]
    inp = ti.make_inputs(cfg)
    c = W.make_config(cfg)
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    half = cfg.seq_len // 2
    out1, out2 = torch.empty_like(q), torch.empty_like(q)
    s1 = W.ttt_init_state(c, w0)
    W.ttt_sequence_forward(s1, q, k, v, eta, out1, cfg.seq_len)
    s2 = W.ttt_init_state(c, w0)
    first = lambda x: x[:, :, :half].contiguous()
    second = lambda x: x[:, :, half:].contiguous()
    o_a, o_b = torch.empty_like(first(q)), torch.empty_like(second(q))
    W.ttt_sequence_forward(s2, first(q), first(k), first(v), first(eta), o_a, half)
    _, flat = read_state(c, s2)
    saved = flat.clone()
    s2.destroy()
    s3 = W.ttt_init_state(c, w0)
    W.ttt_set_state(s3, saved)
    W.ttt_sequence_forward(s3, second(q), second(k), second(v), second(eta), o_b, half)
    torch.cuda.synchronize()
    W1, _ = read_state(c, s1)
    W3, _ = read_state(c, s3)
    assert np.array_equal(out1[:, :, half:].view(torch.int16).cpu().numpy(),
                          o_b.view(torch.int16).cpu().numpy())
    assert all(np.array_equal(a, b) for a, b in zip(W1, W3))
    s1.destroy()
    s3.destroy()


def test_momentum_with_chunks_that_do_not_update():
    cfg = CASES["swiglu_muon_bf16"]
    inp = ti.make_inputs(cfg)
    flags = (1, 0, 0, 1)
    c = W.make_config(cfg)
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    out = torch.empty_like(q)
    st = W.ttt_init_state(c, w0)
    W.ttt_sequence_forward_masked(st, q, k, v, eta, out, cfg.seq_len, flags)
    Ws, _ = read_state(c, st)
    st.destroy()
    O = out.float().cpu().numpy()
    ref = orc.forward_all(cfg, inp, update_chunks=flags)
    for (b, h), (Or, Wr) in ref.items():
        eo = np.abs(O[b, h] - Or).max() / np.abs(Or).max()
        ew = max(np.abs(Ws[m][b, h] - Wr[m]).max() / np.abs(Wr[m]).max() for m in range(len(Wr)))
        assert eo <= 2e-2 and ew <= 2e-2, (b, h, eo, ew)
