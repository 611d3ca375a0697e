"""Replayed forward calls (ttt_config.replay): the first call with given pointers records a
HIP graph, later calls with the same pointers replay it.  Every replay is checked, bit for
bit, against a state that launches directly and sees the same inputs; between the calls the
test does eager work of its own (new inputs copied into the same tensors, unrelated torch
kernels, synchronisations)."""
import numpy as np
import pytest
import torch

import ttt_inputs as ti
import weight_sequence_layers_amd as W
from ttt_gpu import device_inputs, read_state

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_fp32": (ti.CONFIGS["tiny"], None),
    "tiny_shape_muon_bf16": (ti.Config("rp_b", 1, 2, 2048, 256, 64, 128, "swiglu", "dot", 5, True,
                                       "bf16", "apply_then_update", 101), (1, 3, 3, 0)),
    "small_chunk_resident": (ti.Config("rp_c", 2, 3, 1024, 64, 64, 256, "gelu", "mse", 0, False,
                                       "bf16", "apply_then_update", 102), (1, 1, 1, 0)),
    "gelu_mse_fp32": (ti.Config("rp_d", 1, 2, 768, 256, 80, 176, "gelu", "mse", 0, True, "f32",
                                "apply_then_update", 103), None),
}


def _raw(cfg, t):
    return t.view(torch.int16).cpu().numpy() if cfg.act == "bf16" else t.cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_replay_equals_direct_launches(name):
    cfg, planes = CASES[name]
    direct = W.make_config(cfg, planes=planes, replay=False)
    replay = W.make_config(cfg, planes=planes, replay=True)
    inp = ti.make_inputs(cfg)
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    out_d, out_r = torch.empty_like(q), torch.empty_like(q)
    sd, sr = W.ttt_init_state(direct, w0), W.ttt_init_state(replay, w0)
    scratch = torch.zeros(1 << 20, device="cuda")
    for rep in range(4):
        if rep:
            # new inputs in the same tensors, and eager work between the calls
            nxt = ti.make_inputs(cfg, seed=cfg.seed + 17 * rep)
            q2, k2, v2, e2, _ = device_inputs(cfg, nxt)
            q.copy_(q2); k.copy_(k2); v.copy_(v2); eta.copy_(e2)
            scratch.add_(1.0).mul_(0.5)
            torch.cuda.synchronize()
        W.ttt_sequence_forward(sd, q, k, v, eta, out_d, cfg.seq_len)
        W.ttt_sequence_forward(sr, q, k, v, eta, out_r, cfg.seq_len)
        torch.cuda.synchronize()
        Wd, _ = read_state(direct, sd)
        Wr, _ = read_state(replay, sr)
        assert np.array_equal(_raw(cfg, out_d), _raw(cfg, out_r)), (name, rep)
        assert all(np.array_equal(a, b) for a, b in zip(Wd, Wr)), (name, rep)
    W.ttt_state_health(sr)
    sd.destroy()
    sr.destroy()


def test_replay_chunk_api_equals_sequence_api():
    cfg, planes = CASES["tiny_shape_muon_bf16"]
    inp = ti.make_inputs(cfg)
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    b = cfg.chunk
    c = W.make_config(cfg, planes=planes, replay=True)
    s1, s2 = W.ttt_init_state(c, w0), W.ttt_init_state(c, w0)
    out = torch.empty_like(q)
    W.ttt_sequence_forward(s1, q, k, v, eta, out, cfg.seq_len)
    # one set of chunk tensors reused for every chunk: each call after the first replays
    qc, kc, vc = (torch.empty_like(x[:, :, :b]).contiguous() for x in (q, k, v))
    ec = torch.empty_like(eta[:, :, :b]).contiguous()
    oc = torch.empty_like(qc)
    outc = torch.empty_like(q)
    for ci in range(cfg.seq_len // b):
        sl = slice(ci * b, (ci + 1) * b)
        qc.copy_(q[:, :, sl]); kc.copy_(k[:, :, sl]); vc.copy_(v[:, :, sl]); ec.copy_(eta[:, :, sl])
        W.ttt_chunk_forward(s2, qc, kc, vc, ec, oc)
        outc[:, :, sl] = oc
    torch.cuda.synchronize()
    W1, _ = read_state(c, s1)
    W2, _ = read_state(c, s2)
    assert np.array_equal(out.view(torch.int16).cpu().numpy(), outc.view(torch.int16).cpu().numpy())
    assert all(np.array_equal(a, b) for a, b in zip(W1, W2))
    s1.destroy()
    s2.destroy()


def test_replay_with_update_flags_and_new_flags():
    cfg, planes = CASES["tiny_shape_muon_bf16"]
    inp = ti.make_inputs(cfg)
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    outs = {}
    for replay in (False, True):
        c = W.make_config(cfg, planes=planes, replay=replay)
        st = W.ttt_init_state(c, w0)
        res = []
        for flags in ([1, 0] * 4, [1, 0] * 4, [0, 1] * 4, [1, 0] * 4):
            out = torch.empty_like(q) if not res else res[-1][0]
            W.ttt_sequence_forward_masked(st, q, k, v, eta, out, cfg.seq_len, flags)
            torch.cuda.synchronize()
            res.append((out, out.view(torch.int16).cpu().numpy().copy(), read_state(c, st)[0]))
        outs[replay] = res
        st.destroy()
    for (_, o1, w1), (_, o2, w2) in zip(outs[False], outs[True]):
        assert np.array_equal(o1, o2)
        assert all(np.array_equal(a, b) for a, b in zip(w1, w2))
