"""GPU parity of the apply-step backward (ttt_apply_backward) against the oracle's
apply_vjp: dq and every matrix of dw, max relative error per tensor, 1e-4 for fp32
activations and 2e-2 for bf16, at the initial state and after one forward chunk (the
oracle takes its own state after that chunk). dO is the seeded values tensor."""
import numpy as np
import pytest
import torch

import oracle.ttt_oracle as orc
import ttt_inputs as ti
import weight_sequence_layers_amd as W
from ttt_gpu import DEV, device_inputs, rel_err

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _oracle_state(cfg, inp, b, h, n_chunks):
    W0s = [w[h] for w in inp["w0"]]
    if n_chunks == 0:
        return [np.asarray(w, np.float64) for w in W0s]
    _, Ws = orc.sequence_forward(cfg, W0s, inp["q"][b, h], inp["k"][b, h], inp["v"][b, h],
                                 inp["eta"][b, h], n_chunks=n_chunks)
    return Ws


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("fw,loss,ns,renorm", [
    ("swiglu", "dot", 5, True), ("gelu", "mse", 0, False), ("linear", "dot", 0, False),
])
def test_apply_backward_parity(act, fw, loss, ns, renorm):
    cfg = ti.Config("bwd", 2, 2, 600, 300, 80, 176, fw, loss, ns, renorm, act,
                    "apply_then_update", 61)
    inp = ti.make_inputs(cfg)
    c = W.make_config(cfg, path="staged")
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    st = W.ttt_init_state(c, w0)
    n = W.ttt_state_numel(c)
    b = cfg.chunk
    tol = TOL[act]
    for ci in range(2):
        sl = slice(ci * b, (ci + 1) * b)
        qc, dout = q[:, :, sl].contiguous(), v[:, :, sl].contiguous()
        dq = torch.empty_like(qc)
        dw = torch.empty(n, dtype=torch.float32, device=DEV)
        W.ttt_apply_backward(st, qc, dout, dq, dw)
        torch.cuda.synchronize()
        dq_g = dq.float().cpu().numpy()
        dw_g = [x.cpu().numpy() for x in W.split_state(c, dw)]
        worst = 0.0
        for bb in range(cfg.batch):
            for h in range(cfg.heads):
                Ws = _oracle_state(cfg, inp, bb, h, ci)
                dQ, dWs = orc.apply_vjp(fw, Ws, inp["q"][bb, h, sl], inp["v"][bb, h, sl])
                errs = [rel_err(dq_g[bb, h], dQ)] + [rel_err(g[bb, h], r)
                                                     for g, r in zip(dw_g, dWs)]
                worst = max(worst, max(errs))
                assert max(errs) <= tol, (ci, bb, h, errs)
        print(f"{fw} {act} chunk {ci}: max rel err {worst:.3e} (tol {tol})", flush=True)
        if ci == 0:
            out = torch.empty_like(qc)
            W.ttt_chunk_forward(st, qc, k[:, :, sl].contiguous(), dout,
                                eta[:, :, sl].contiguous(), out)
    W.ttt_state_health(st)
    st.destroy()


def test_apply_backward_rejects_resident_states():
    cfg = ti.Config("bwdres", 1, 2, 64, 64, 64, 256, "gelu", "mse", 0, False, "bf16",
                    "apply_then_update", 62)
    c = W.make_config(cfg, planes=(1, 1, 1, 0), path="resident")
    inp = ti.make_inputs(cfg)
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    st = W.ttt_init_state(c, w0)
    dq = torch.empty_like(q)
    dw = torch.empty(W.ttt_state_numel(c), dtype=torch.float32, device=DEV)
    with pytest.raises(W.TTTError) as e:
        W.ttt_apply_backward(st, q, v, dq, dw)
    assert e.value.status == 5
    st.destroy()


def _backward_vs_oracle(cfg, problems, planes=None):
    inp = ti.make_inputs(cfg)
    c = W.make_config(cfg, planes=planes, path="staged")
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    st = W.ttt_init_state(c, w0)
    b = cfg.chunk
    qc, dout = q[:, :, :b].contiguous(), v[:, :, :b].contiguous()
    dq = torch.empty_like(qc)
    dw = torch.empty(W.ttt_state_numel(c), dtype=torch.float32, device=DEV)
    W.ttt_apply_backward(st, qc, dout, dq, dw)
    torch.cuda.synchronize()
    dq_g = dq.float().cpu().numpy()
    dw_g = [x.cpu().numpy() for x in W.split_state(c, dw)]
    st.destroy()
    worst = 0.0
    for bb, h in problems:
        dQ, dWs = orc.apply_vjp(cfg.fw, [w[h] for w in inp["w0"]], inp["q"][bb, h, :b],
                                inp["v"][bb, h, :b])
        errs = [rel_err(dq_g[bb, h], dQ)] + [rel_err(g[bb, h], r) for g, r in zip(dw_g, dWs)]
        worst = max(worst, max(errs))
    print(f"{cfg.name}: apply backward max rel err {worst:.3e}", flush=True)
    return worst


def test_apply_backward_lm_full_size():
    # the LM layer's chunk (2048 tokens, 8 problems, dim 512, hidden 1024) in its preset
    cfg = ti.CONFIGS["lm"].replace(seq_len=2048)
    assert _backward_vs_oracle(cfg, [(0, 0), (3, 1)]) <= TOL["bf16"]


def test_apply_backward_chunk_longer_than_a_block():
    # 140000 tokens: blocks of 65536, 65536 and 8928 whose weight gradients accumulate
    cfg = ti.Config("bwdlong", 1, 1, 140000, 140000, 64, 128, "swiglu", "dot", 5, True,
                    "bf16", "update_then_apply", 63)
    assert _backward_vs_oracle(cfg, [(0, 0)]) <= TOL["bf16"]


def test_apply_backward_leaves_state_and_is_linear_in_dout_bitwise():
    # the state is not touched; dO scaled by 2 (exact in bf16) scales dq and dw by exactly 2
    cfg = ti.Config("bwdinv", 2, 2, 256, 256, 80, 176, "swiglu", "dot", 5, True, "bf16",
                    "apply_then_update", 64)
    inp = ti.make_inputs(cfg)
    c = W.make_config(cfg, path="staged")
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    st = W.ttt_init_state(c, w0)
    n = W.ttt_state_numel(c)
    before = torch.empty(n, dtype=torch.float32, device=DEV)
    after = torch.empty_like(before)
    W.ttt_get_state(st, before)
    res = []
    for scale in (1.0, 2.0):
        dout = (v * scale).contiguous()
        dq = torch.empty_like(q)
        dw = torch.empty(n, dtype=torch.float32, device=DEV)
        W.ttt_apply_backward(st, q, dout, dq, dw)
        res.append((dq.float().cpu(), dw.cpu()))
    W.ttt_get_state(st, after)
    torch.cuda.synchronize()
    st.destroy()
    assert torch.equal(before, after)
    assert torch.equal(res[1][0], 2.0 * res[0][0])
    assert torch.equal(res[1][1], 2.0 * res[0][1])


def test_apply_backward_argument_checks():
    # null and misaligned pointers are refused on the host, before anything is enqueued
    cfg = ti.Config("bwdarg", 1, 1, 64, 64, 64, 128, "swiglu", "dot", 0, False, "f32",
                    "apply_then_update", 65)
    inp = ti.make_inputs(cfg)
    c = W.make_config(cfg, path="staged")
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    st = W.ttt_init_state(c, w0)
    dq = torch.empty_like(q)
    dw = torch.empty(W.ttt_state_numel(c) + 4, dtype=torch.float32, device=DEV)
    L = W.lib()
    assert L.ttt_apply_backward(st.handle, q.data_ptr(), v.data_ptr(), None, dw.data_ptr(),
                                None) == 1
    assert L.ttt_apply_backward(st.handle, q.data_ptr(), v.data_ptr(), dq.data_ptr(),
                                dw.data_ptr() + 4, None) == 9
    assert L.ttt_apply_backward(None, q.data_ptr(), v.data_ptr(), dq.data_ptr(),
                                dw.data_ptr(), None) == 1
    W.ttt_apply_backward(st, q, v, dq, dw[:W.ttt_state_numel(c)])
    torch.cuda.synchronize()
    st.destroy()
