"""Helpers shared by the GPU tests: upload seeded inputs, run libttt through its binding,
read results back, and measure errors against the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle.ttt_oracle as orc
import ttt_inputs as ti
import weight_sequence_layers_amd as W

DEV = "cuda"


def to_device(cfg, arr_vals, arr_bits=None):
    if cfg.act == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr_bits).view(np.int16)).to(DEV).view(
            torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr_vals)).to(DEV)


def device_inputs(cfg, inp):
    q = to_device(cfg, inp["q"], inp.get("q_bits"))
    k = to_device(cfg, inp["k"], inp.get("k_bits"))
    v = to_device(cfg, inp["v"], inp.get("v_bits"))
    eta = torch.from_numpy(np.ascontiguousarray(inp["eta"])).to(DEV)
    w0 = torch.from_numpy(np.concatenate([w.ravel() for w in inp["w0"]])).to(DEV)
    return q, k, v, eta, w0


def read_state(c, st):
    flat = torch.empty(W.ttt_state_numel(c), dtype=torch.float32, device=DEV)
    W.ttt_get_state(st, flat)
    torch.cuda.synchronize()
    return [w.cpu().numpy().astype(np.float64) for w in W.split_state(c, flat)], flat


def run_gpu(cfg, inp, planes=None, chunked=False, path="auto", launches=None):
    """Whole sequence through libttt. Returns (O [B,H,T,d] fp32, [W per matrix [B,H,r,c]]).
    launches: optional stage name; its launch count is appended to `launches_out`."""
    c = W.make_config(cfg, planes=planes, path=path)
    q, k, v, eta, w0 = device_inputs(cfg, inp)
    out = torch.empty_like(q)
    st = W.ttt_init_state(c, w0)
    if launches is not None:
        W.ttt_profile_begin(st, launches[0], 1 << 16)
    if chunked:
        b = cfg.chunk
        for ci in range(cfg.seq_len // b):
            sl = slice(ci * b, (ci + 1) * b)
            qc, kc, vc = q[:, :, sl].contiguous(), k[:, :, sl].contiguous(), v[:, :, sl].contiguous()
            ec = eta[:, :, sl].contiguous()
            oc = torch.empty_like(qc)
            W.ttt_chunk_forward(st, qc, kc, vc, ec, oc)
            out[:, :, sl] = oc
    else:
        W.ttt_sequence_forward(st, q, k, v, eta, out, cfg.seq_len)
    if launches is not None:
        launches.append(W.ttt_profile_end(st)[0])
    Ws, _ = read_state(c, st)
    W.ttt_state_health(st)
    O = out.float().cpu().numpy()
    st.destroy()
    return O, Ws


def rel_err(x, y) -> float:
    den = float(np.abs(y).max())
    return float(np.abs(x - y).max()) / (den if den > 0 else 1.0)


def oracle_all(cfg, inp, problems=None, block_rows=8192):
    return orc.forward_all(cfg, inp, problems, block_rows)


def parity(cfg, inp, O, Ws, problems=None):
    """Max relative errors (O, [W_m]) of the GPU result against the oracle over the listed
    (batch, head) problems (all by default)."""
    ref = oracle_all(cfg, inp, problems)
    probs = list(ref.keys())
    Og = np.stack([O[b, h] for b, h in probs])
    Or = np.stack([ref[p][0] for p in probs])
    errs_w = []
    for m in range(len(Ws)):
        Wg = np.stack([Ws[m][b, h] for b, h in probs])
        Wr = np.stack([ref[p][1][m] for p in probs])
        errs_w.append(rel_err(Wg, Wr))
    return rel_err(Og, Or), errs_w


def small(name, **kw):
    return ti.CONFIGS[name].replace(**kw)
