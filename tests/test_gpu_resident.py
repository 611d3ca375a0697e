"""GPU tests of the device-resident chunk loop (one kernel per call; the small-chunk GELU-MLP
layer with plain gradient steps): parity with the oracle on full chunks, ragged chunks
(chunk < 64 leaves padded rows), single-token chunks and the inner-product loss; agreement
with the staged kernels; and the bitwise invariants (chunk API = sequence API, eta = 0,
determinism, NaN flag). Errors are max relative errors |x - y|_inf / |y|_inf over all
compared values; the bound for bf16 activations with one bf16 plane is 2e-2."""
import numpy as np
import pytest
import torch

import oracle.ttt_oracle as orc
import ttt_inputs as ti
import weight_sequence_layers_amd as W
from ttt_gpu import parity, run_gpu

pytestmark = pytest.mark.gpu

TOL = 2e-2
PLANES = (1, 1, 1, 1)
BASE = ti.Config("resident", 2, 3, 768, 64, 64, 256, "gelu", "mse", 0, False, "bf16",
                 "apply_then_update", 2024)


def _resident(cfg, inp, **kw):
    n = ["resident"]
    O, Ws = run_gpu(cfg, inp, PLANES, path="resident", launches=n, **kw)
    assert n[1] == (1 if not kw.get("chunked") else cfg.seq_len // cfg.chunk), n
    return O, Ws


@pytest.mark.parametrize("name,kw", [
    ("mse chunk 64", {}),
    ("mse chunk 48 (padded rows)", {"chunk": 48, "seq_len": 480}),
    ("mse chunk 1", {"chunk": 1, "seq_len": 40}),
    ("mse chunk 17", {"chunk": 17, "seq_len": 17 * 9}),
    ("dot loss chunk 64", {"loss": "dot"}),
    ("one problem, one chunk", {"batch": 1, "heads": 1, "seq_len": 64}),
    ("mse, step sizes and decay", {"lr": (0.5, 1.8), "weight_decay": 0.03}),
    ("dot, step sizes and decay", {"loss": "dot", "lr": (2.0, 0.25), "weight_decay": 0.1,
                                   "chunk": 33, "seq_len": 33 * 7}),
])
def test_resident_parity(name, kw):
    cfg = BASE.replace(**kw)
    inp = ti.make_inputs(cfg)
    O, Ws = _resident(cfg, inp)
    eo, ew = parity(cfg, inp, O, Ws)
    print(f"{name}: O {eo:.3e} W {[f'{e:.3e}' for e in ew]}", flush=True)
    assert eo <= TOL and max(ew) <= TOL, (name, eo, ew)


def test_resident_matches_staged():
    cfg = BASE
    inp = ti.make_inputs(cfg)
    O1, W1 = _resident(cfg, inp)
    O2, W2 = run_gpu(cfg, inp, PLANES, path="staged")
    d = float(np.abs(O1 - O2).max() / np.abs(O2).max())
    dw = [float(np.abs(a - b).max() / np.abs(b).max()) for a, b in zip(W1, W2)]
    print(f"resident vs staged: O {d:.3e} W {dw}", flush=True)
    assert d <= TOL and max(dw) <= TOL


def test_resident_chunk_api_equals_sequence_api_bitwise():
    cfg = BASE.replace(seq_len=256)
    inp = ti.make_inputs(cfg)
    O1, W1 = _resident(cfg, inp)
    O2, W2 = _resident(cfg, inp, chunked=True)
    assert np.array_equal(O1, O2)
    for a, b in zip(W1, W2):
        assert np.array_equal(a, b)


def test_resident_deterministic_bitwise():
    cfg = BASE.replace(seq_len=256)
    inp = ti.make_inputs(cfg)
    O1, W1 = _resident(cfg, inp)
    O2, W2 = _resident(cfg, inp)
    assert np.array_equal(O1, O2)
    for a, b in zip(W1, W2):
        assert np.array_equal(a, b)


def test_resident_eta_zero_keeps_state_bitwise():
    cfg = BASE.replace(seq_len=256)
    inp = ti.make_inputs(cfg)
    inp["eta"] = np.zeros_like(inp["eta"])
    O, Ws = _resident(cfg, inp)
    for m, w0 in enumerate(inp["w0"]):
        for b in range(cfg.batch):
            assert np.array_equal(Ws[m][b], w0.astype(np.float64)), (m, b)
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            ref = orc.fw_apply(cfg.fw, [w[h] for w in inp["w0"]], inp["q"][b, h])
            assert np.abs(O[b, h] - ref).max() <= TOL * np.abs(ref).max()


def test_resident_nan_sets_health_flag():
    cfg = BASE.replace(batch=1, heads=1, seq_len=128)
    inp = ti.make_inputs(cfg)
    inp["eta"][0, 0, 70] = np.nan
    c = W.make_config(cfg, planes=PLANES, path="resident")
    from ttt_gpu import device_inputs
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    out = torch.empty_like(q)
    st = W.ttt_init_state(c, w0)
    W.ttt_sequence_forward(st, q, k, v, eta, out, cfg.seq_len)
    with pytest.raises(W.TTTError) as e:
        W.ttt_state_health(st)
    assert "NaN" in str(e.value) or "finite" in str(e.value)
    st.destroy()


def test_auto_path_picks_resident_for_small_chunk_layer():
    cfg = BASE.replace(batch=1, heads=2, seq_len=128)
    inp = ti.make_inputs(cfg)
    n = ["resident"]
    run_gpu(cfg, inp, PLANES, path="auto", launches=n)
    assert n[1] == 1
