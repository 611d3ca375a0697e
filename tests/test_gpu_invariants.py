"""GPU invariants of libttt that must hold bit for bit, plus edge cases: eta = 0, the chunk
API against the sequence API, resume through get/set, run-to-run determinism, shifted
causality, NaN detection, empty sequences, multi-block chunks and many problems."""
import numpy as np
import pytest
import torch

import oracle.ttt_oracle as orc
import ttt_inputs as ti
import weight_sequence_layers_amd as W
from ttt_gpu import device_inputs, parity, read_state, run_gpu

pytestmark = pytest.mark.gpu

CFG = ti.Config("inv", 2, 2, 1280, 256, 64, 128, "swiglu", "dot", 5, True, "bf16",
                "apply_then_update", 99)


def _run(cfg, inp, planes=None, chunked=False):
    return run_gpu(cfg, inp, planes, chunked)


def test_eta_zero_keeps_state_bitwise():
    for cfg in (CFG, CFG.replace(fw="gelu", loss="mse", ns_steps=0, renorm=False),
                CFG.replace(act="f32")):
        inp = ti.make_inputs(cfg)
        inp["eta"] = np.zeros_like(inp["eta"])
        O, Ws = _run(cfg, inp)
        for m, w0 in enumerate(inp["w0"]):
            for b in range(cfg.batch):
                assert np.array_equal(Ws[m][b], w0.astype(np.float64)), (cfg.fw, m, b)
        # and the outputs are the initial net applied to the queries
        for b in range(cfg.batch):
            for h in range(cfg.heads):
                ref = orc.fw_apply(cfg.fw, [w[h] for w in inp["w0"]], inp["q"][b, h])
                tol = 1e-4 if cfg.act == "f32" else 2e-2
                assert np.abs(O[b, h] - ref).max() <= tol * np.abs(ref).max()


def test_chunk_api_equals_sequence_api_bitwise():
    inp = ti.make_inputs(CFG)
    O1, W1 = _run(CFG, inp)
    O2, W2 = _run(CFG, inp, chunked=True)
    assert np.array_equal(O1, O2)
    for a, b in zip(W1, W2):
        assert np.array_equal(a, b)


def test_deterministic_bitwise():
    inp = ti.make_inputs(CFG)
    O1, W1 = _run(CFG, inp)
    O2, W2 = _run(CFG, inp)
    assert np.array_equal(O1, O2)
    for a, b in zip(W1, W2):
        assert np.array_equal(a, b)


def test_resume_through_get_set_state_bitwise():
    cfg = CFG
    inp = ti.make_inputs(cfg)
    O_ref, W_ref = _run(cfg, inp)
    c = W.make_config(cfg)
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    half = 2 * cfg.chunk
    out = torch.empty_like(q)
    st = W.ttt_init_state(c, w0)
    sl = slice(0, half)
    part = [x[:, :, sl].contiguous() for x in (q, k, v, eta)]
    o1 = torch.empty_like(part[0])
    W.ttt_sequence_forward(st, *part, o1, half)
    _, flat = read_state(c, st)
    st.destroy()
    st2 = W.ttt_init_state(c, w0)         # fresh state, then overwrite with the snapshot
    W.ttt_set_state(st2, flat)
    sl = slice(half, cfg.seq_len)
    part = [x[:, :, sl].contiguous() for x in (q, k, v, eta)]
    o2 = torch.empty_like(part[0])
    W.ttt_sequence_forward(st2, *part, o2, cfg.seq_len - half)
    Ws, _ = read_state(c, st2)
    st2.destroy()
    O = torch.cat([o1, o2], dim=2).float().cpu().numpy()
    assert np.array_equal(O, O_ref)
    for a, b in zip(Ws, W_ref):
        assert np.array_equal(a, b)


def test_shifted_causality_bitwise():
    cfg = CFG
    inp = ti.make_inputs(cfg)
    O_ref, _ = _run(cfg, inp)
    b = cfg.chunk
    for c in (0, 2):
        pert = {k: (x.copy() if isinstance(x, np.ndarray) else x) for k, x in inp.items()}
        lo = c * b
        pert["eta"][:, :, lo:] *= 2.0
        kv, _ = ti.bf16_round(pert["k"][:, :, lo:] * -1.0)
        pert["k"][:, :, lo:] = kv
        pert["k_bits"][:, :, lo:] = ti.bf16_round(kv)[1]
        O, _ = _run(cfg, pert)
        assert np.array_equal(O[:, :, :lo + b], O_ref[:, :, :lo + b])
        assert not np.array_equal(O[:, :, lo + b:], O_ref[:, :, lo + b:])


def test_nonfinite_values_are_reported():
    cfg = CFG.replace(ns_steps=0)
    inp = ti.make_inputs(cfg)
    inp["v"][1, 0, 300] = np.nan
    inp["v_bits"][1, 0, 300] = 0x7FC0
    c = W.make_config(cfg)
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    out = torch.empty_like(q)
    st = W.ttt_init_state(c, w0)
    W.ttt_sequence_forward(st, q, k, v, eta, out, cfg.seq_len)
    with pytest.raises(W.TTTError) as e:
        W.ttt_state_health(st)
    assert e.value.status == 8
    # set_state clears the flag
    W.ttt_set_state(st, w0.new_zeros(W.ttt_state_numel(c)) + 0.5)
    W.ttt_state_health(st)
    st.destroy()


def test_empty_sequence_and_shape_errors():
    cfg = CFG
    inp = ti.make_inputs(cfg.replace(seq_len=cfg.chunk))
    c = W.make_config(cfg)
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    out = torch.empty_like(q)
    st = W.ttt_init_state(c, w0)
    W.ttt_sequence_forward(st, q, k, v, eta, out, 0)            # no-op
    Ws, _ = read_state(c, st)
    for m, w in enumerate(inp["w0"]):
        assert np.array_equal(Ws[m][0], w.astype(np.float64))
    with pytest.raises(W.TTTError) as e:
        W.ttt_sequence_forward(st, q, k, v, eta, out, cfg.chunk + 1)
    assert e.value.status == 2
    with pytest.raises(W.TTTError) as e:
        W.ttt_sequence_forward(st, q, k, v, None, out, cfg.chunk)
    assert e.value.status == 1
    st.destroy()


def test_chunk_longer_than_one_token_block():
    """A chunk of 70000 tokens is summed over two token blocks of the gradient launch."""
    cfg = ti.Config("long_chunk", 1, 1, 70000, 70000, 16, 32, "swiglu", "dot", 5, True, "bf16",
                    "update_then_apply", 5)
    inp = ti.make_inputs(cfg)
    O, Ws = _run(cfg, inp, planes=(1, 2, 2, 0))
    eo, ew = parity(cfg, inp, O, Ws)
    assert eo <= 2e-2 and max(ew) <= 2e-2, (eo, ew)


def test_many_problems():
    cfg = ti.Config("many", 30, 10, 96, 48, 16, 32, "gelu", "mse", 0, False, "bf16",
                    "apply_then_update", 6)
    inp = ti.make_inputs(cfg)
    O, Ws = _run(cfg, inp)
    eo, ew = parity(cfg, inp, O, Ws, problems=[(0, 0), (17, 3), (29, 9)])
    assert eo <= 2e-2 and max(ew) <= 2e-2, (eo, ew)


def test_single_token_chunks():
    cfg = ti.Config("tok", 1, 2, 24, 1, 32, 64, "swiglu", "mse", 0, True, "f32",
                    "apply_then_update", 8)
    inp = ti.make_inputs(cfg)
    O, Ws = _run(cfg, inp)
    eo, ew = parity(cfg, inp, O, Ws)
    assert eo <= 1e-4 and max(ew) <= 1e-4, (eo, ew)
