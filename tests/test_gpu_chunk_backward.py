"""GPU parity of the backward through one chunk (ttt_chunk_backward) against the oracle's
chunk_vjp on the same seeded inputs and cotangents: the input gradients dq, dk, dv, deta
and the state cotangent before the chunk, for the SwiGLU net with the inner-product loss,
under both orders, with and without Muon and the row renorm, with step sizes, weight decay
and momentum, fp32 and bf16,
at ragged small sizes, at the LaCT language-model chunk, and chained over a short sequence
(each call from the state before its chunk; a chunk that does not update taken back by the
apply backward alone).  Errors are max relative errors
|x - y|_inf / |y|_inf per tensor; bars 1e-4 (fp32) and 2e-2 (bf16)."""
import numpy as np
import pytest
import torch

import oracle.ttt_oracle as orc
import ttt_inputs as ti
import weight_sequence_layers_amd as W
from ttt_gpu import device_inputs, read_state, rel_err, to_device

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _cotangents(cfg, seed):
    """dO (activation dtype values, as the device receives them) and dW_after (fp32, state
    layout), seeded."""
    rng = np.random.default_rng(seed)
    dO = rng.standard_normal((cfg.batch, cfg.heads, cfg.seq_len, cfg.dim)).astype(np.float32)
    bits = None
    if cfg.act == "bf16":
        dO, bits = ti.bf16_round(dO)
    shapes = cfg.matrix_shapes() * (2 if cfg.momentum else 1)   # with the momentum buffers
    dWs = [rng.standard_normal((cfg.batch, cfg.heads) + s).astype(np.float32) for s in shapes]
    return dO, bits, dWs


def _gpu_backward(cfg, inp, dO, bits, dWs, planes=None, update=None):
    """ttt_chunk_backward over the chunks of the sequence, last to first, each from the
    state before its chunk (taken during a forward pass with ttt_get_state). update: one
    flag per chunk; a chunk that does not update is answered by ttt_sequence_forward_masked
    and taken back by ttt_apply_backward, its weight gradient added to the state's
    cotangent (its keys, values and step sizes get none)."""
    c = W.make_config(cfg, planes=planes, path="staged")
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    st = W.ttt_init_state(c, w0)
    b = cfg.chunk
    nc = cfg.seq_len // b
    states = []
    out = torch.empty_like(q[:, :, :b]).contiguous()
    sl = lambda x, ci: x[:, :, ci * b:(ci + 1) * b].contiguous()
    up = [True] * nc if update is None else [bool(u) for u in update]
    for ci in range(nc):
        _, flat = read_state(c, st)
        states.append(flat.clone())
        if up[ci]:
            W.ttt_chunk_forward(st, sl(q, ci), sl(k, ci), sl(v, ci), sl(eta, ci), out)
        else:
            W.ttt_sequence_forward_masked(st, sl(q, ci), sl(k, ci), sl(v, ci), sl(eta, ci),
                                          out, b, [False])
    dw = torch.from_numpy(np.concatenate([x.ravel() for x in dWs])).cuda()
    dOd = to_device(cfg, dO, bits)
    res = {n: np.zeros((cfg.batch, cfg.heads, cfg.seq_len, cfg.dim)) for n in ("dq", "dk", "dv")}
    res["deta"] = np.zeros((cfg.batch, cfg.heads, cfg.seq_len))
    for ci in reversed(range(nc)):
        W.ttt_set_state(st, states[ci])
        g = {n: torch.empty_like(sl(q, ci)) for n in ("dq", "dk", "dv")}
        deta = torch.empty_like(sl(eta, ci))
        if up[ci]:
            W.ttt_chunk_backward(st, sl(q, ci), sl(k, ci), sl(v, ci), sl(eta, ci), sl(dOd, ci),
                                 dw, g["dq"], g["dk"], g["dv"], deta)
        else:
            dwa = torch.empty_like(dw)
            W.ttt_apply_backward(st, sl(q, ci), sl(dOd, ci), g["dq"], dwa)
            dw += dwa
            for n in ("dk", "dv"):
                g[n].zero_()
            deta.zero_()
        torch.cuda.synchronize()
        for n in ("dq", "dk", "dv"):
            res[n][:, :, ci * b:(ci + 1) * b] = g[n].float().cpu().numpy()
        res["deta"][:, :, ci * b:(ci + 1) * b] = deta.cpu().numpy()
    W.ttt_state_health(st)
    res["dw"] = [x.cpu().numpy().astype(np.float64) for x in W.split_state(c, dw)]
    st.destroy()
    return res


def _check(cfg, planes=None, problems=None, seed=5, update=None):
    inp = ti.make_inputs(cfg)
    dO, bits, dWs = _cotangents(cfg, seed)
    got = _gpu_backward(cfg, inp, dO, bits, dWs, planes, update)
    tol = TOL[cfg.act]
    probs = problems or [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    worst = 0.0
    for (b, h) in probs:
        W0s = [w[h] for w in inp["w0"]]
        ref = orc.sequence_vjp(cfg, W0s, inp["q"][b, h], inp["k"][b, h], inp["v"][b, h],
                               inp["eta"][b, h], dO[b, h], [x[b, h] for x in dWs], update)
        errs = {n: rel_err(got[n][b, h], r) for n, r in zip(("dq", "dk", "dv", "deta"), ref[:4])}
        errs.update({f"dW{m}": rel_err(got["dw"][m][b, h], r) for m, r in enumerate(ref[4])})
        print(f"{cfg.name} problem ({b},{h}): " +
              " ".join(f"{n} {e:.2e}" for n, e in errs.items()), flush=True)
        worst = max(worst, max(errs.values()))
        assert max(errs.values()) <= tol, errs
    return worst


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("ns,renorm", [(0, False), (0, True), (5, True)])
def test_chunk_backward_small(act, ns, renorm):
    cfg = ti.Config("cb", 2, 2, 300, 300, 80, 176, "swiglu", "dot", ns, renorm, act,
                    "apply_then_update", 91)
    _check(cfg)


def test_chunk_backward_step_size_and_decay():
    cfg = ti.Config("cbl", 1, 2, 256, 256, 64, 128, "swiglu", "dot", 5, True, "f32",
                    "apply_then_update", 92, lr=(0.5, 1.5, 0.8), weight_decay=0.05)
    _check(cfg)


def test_chunk_backward_chained_over_three_chunks():
    cfg = ti.Config("cbs", 1, 2, 384, 128, 64, 128, "swiglu", "dot", 5, True, "f32",
                    "apply_then_update", 93)
    _check(cfg)


@pytest.mark.parametrize("order", ["apply_then_update", "update_then_apply"])
def test_chunk_backward_chained_with_a_chunk_that_does_not_update(order):
    # update flags (1, 0, 1): the middle chunk only answers its queries, and its backward is
    # the apply step's alone
    cfg = ti.Config("cbf", 1, 2, 384, 128, 64, 128, "swiglu", "dot", 5, True, "f32", order, 99)
    _check(cfg, update=(1, 0, 1))


@pytest.mark.parametrize("act,ns,renorm", [("f32", 5, True), ("bf16", 0, True), ("f32", 0, False)])
def test_chunk_backward_update_then_apply(act, ns, renorm):
    # the queries see the updated state: the apply backward at the state after the update,
    # its weight gradient taken back through the update; chained over two chunks, with step
    # sizes and weight decay in the first case
    kw = dict(lr=(0.7, 1.2, 0.9), weight_decay=0.02) if ns else {}
    cfg = ti.Config("cbu2", 2, 1, 256, 128, 64, 128, "swiglu", "dot", ns, renorm, act,
                    "update_then_apply", 95, **kw)
    _check(cfg)


@pytest.mark.parametrize("order,momentum", [("apply_then_update", 0.0),
                                            ("update_then_apply", 0.0),
                                            ("update_then_apply", 0.7)])
def test_chunk_backward_two_token_blocks(order, momentum):
    # a chunk longer than one token block (65536 tokens): the recompute's two contractions
    # keep separate running sums over the blocks (the momentum buffer joins both at the
    # last block), the backward's launches walk the blocks
    cfg = ti.Config("cbb", 1, 1, 66000, 66000, 64, 128, "swiglu", "dot", 5, True, "bf16",
                    order, 97, momentum=momentum)
    _check(cfg)


def test_chunk_backward_lm_chunk():
    # the LaCT language-model layer's shape and precision preset, one chunk of 2048 tokens
    lm = ti.CONFIGS["lm"]
    cfg = lm.replace(name="lm", seq_len=lm.chunk)
    _check(cfg, problems=[(0, 0), (3, 1)])


@pytest.mark.parametrize("act,ns,renorm,order", [
    ("f32", 5, True, "apply_then_update"), ("bf16", 5, True, "update_then_apply"),
    ("f32", 0, False, "update_then_apply"), ("bf16", 0, True, "apply_then_update")])
def test_chunk_backward_momentum(act, ns, renorm, order):
    # heavy-ball buffers in the state: their cotangents in and out, over two chunks, at
    # ragged sizes (the buffers' transposed tiles cut at the matrix edges)
    cfg = ti.Config("cbm", 1, 2, 256, 128, 80, 176, "swiglu", "dot", ns, renorm, act, order,
                    98, lr=(0.8, 1.1, 0.9), weight_decay=0.02, momentum=0.6)
    _check(cfg)


def test_chunk_backward_lm_chunk_momentum():
    # the LaCT language-model layer's shape with heavy-ball momentum, chained over two
    # chunks of 2048 tokens so that the second starts from a buffer that is not zero
    lm = ti.CONFIGS["lm"]
    cfg = lm.replace(name="lmm", seq_len=2 * lm.chunk, momentum=0.9)
    _check(cfg, problems=[(1, 0), (2, 1)])


def test_chunk_backward_refuses_other_configurations():
    for kw in (dict(fw="gelu"), dict(loss="mse", ns_steps=0, renorm=False)):
        cfg = ti.Config("cbu", 1, 1, 128, 128, 64, 128, "swiglu", "dot", 5, True, "bf16",
                        "apply_then_update", 94).replace(**kw)
        c = W.make_config(cfg, path="staged")
        inp = ti.make_inputs(cfg)
        q, k, v, eta, w0 = device_inputs(cfg, inp)
        st = W.ttt_init_state(c, w0)
        dw = torch.zeros(W.ttt_state_numel(c), device="cuda")
        with pytest.raises(W.TTTError) as e:
            W.ttt_chunk_backward(st, q, k, v, eta, q, dw, torch.empty_like(q),
                                 torch.empty_like(q), torch.empty_like(q), torch.empty_like(eta))
        assert e.value.status == 5
        st.destroy()


@pytest.mark.parametrize("order,momentum", [("update_then_apply", 0.0),
                                            ("update_then_apply", 0.5),
                                            ("apply_then_update", 0.5)])
def test_chunk_backward_leaves_the_state(order, momentum):
    # the update-then-apply backward forms the updated state in place of the state and
    # restores it, and both orders read the momentum buffers without replacing them: the
    # state (and its planes, through a forward call) is bitwise unchanged
    cfg = ti.Config("cbu3", 1, 2, 128, 128, 64, 128, "swiglu", "dot", 5, True, "bf16",
                    order, 96, momentum=momentum)
    c = W.make_config(cfg, path="staged")
    inp = ti.make_inputs(cfg)
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    st = W.ttt_init_state(c, w0)
    _, before = read_state(c, st)
    before = before.clone()
    out0 = torch.empty_like(q)
    W.ttt_chunk_forward(st, q, k, v, eta, out0)
    W.ttt_set_state(st, before)
    dw = torch.ones(W.ttt_state_numel(c), device="cuda")
    W.ttt_chunk_backward(st, q, k, v, eta, q, dw, torch.empty_like(q), torch.empty_like(q),
                         torch.empty_like(q), torch.empty_like(eta))
    _, after = read_state(c, st)
    assert torch.equal(after, before)
    out1 = torch.empty_like(q)
    W.ttt_chunk_forward(st, q, k, v, eta, out1)
    torch.cuda.synchronize()
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    st.destroy()
