#!/usr/bin/env python3
"""Throughput of the large-chunk TTT layer forward on one MI355X.

A step is one ttt_sequence_forward over the whole synthetic batch: every chunk's apply,
gradient, Newton-Schulz orthogonalisation, update and row renorm, chunk after chunk. The
state carries over from step to step (the cost of a step does not depend on the state).
Inputs are resident in HBM before the timed region starts.

Prints one JSON line with tokens/s (timed steps with no events), the roofline of the
dominant stage kernel (its algorithmic FLOP per launch over its average launch time, taken
with HIP events on the launch stream over as many steps again, right after the timed ones)
and the CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload lm]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stage_flops(cfg) -> dict:
    """Algorithmic FLOP of each stage per step (the whole sequence, all problems; 2 per
    multiply-add; Newton-Schulz counted without symmetry savings). The resident loop is
    one stage that does everything."""
    P, b, d, dh = cfg.batch * cfg.heads, cfg.chunk, cfg.dim, cfg.hidden
    nz = {"swiglu": 2, "gelu": 1, "linear": 1}[cfg.fw]
    nm = {"swiglu": 3, "gelu": 2, "linear": 1}[cfg.fw]
    n = d if cfg.fw == "linear" else dh
    nc = cfg.n_chunks
    f = {}
    if cfg.fw != "linear":
        f["front_q"] = 2.0 * nz * b * d * dh * P * nc
        f["front_k"] = 2.0 * (nz + (1 if cfg.loss == "dot" else 0)) * b * d * dh * P * nc
        f["out"] = 2.0 * b * d * dh * P * nc
    else:
        f["out"] = 2.0 * b * d * d * P * nc
    f["contract"] = 2.0 * nm * b * d * n * P * nc
    m, it = d, cfg.ns_steps * nc
    f["ns_gram"] = 2.0 * m * m * n * nm * P * it
    f["ns_poly"] = 2.0 * m * m * m * nm * P * it
    f["ns_update"] = 2.0 * m * m * n * nm * P * it
    if ns_small(cfg):   # every iteration in one launch per chunk
        f["ns_small"] = f.pop("ns_gram") + f.pop("ns_poly") + f.pop("ns_update")
    f["resident"] = total_flops(cfg)
    return f


def ns_small(cfg) -> bool:
    """Whether the forward orthogonalises with the fused small-matrix launch (matrices of
    at most 64 x 128 in their [dim][hidden] orientation)."""
    n = cfg.dim if cfg.fw == "linear" else cfg.hidden
    return cfg.ns_steps > 0 and cfg.dim <= 64 and n <= 128


def total_flops(cfg) -> float:
    """Algorithmic FLOP of the whole sequence forward (all problems, all chunks)."""
    d, dh = cfg.dim, cfg.hidden
    per_tok = {("swiglu", "dot"): 18, ("swiglu", "mse"): 20, ("gelu", "dot"): 12,
               ("gelu", "mse"): 14}.get((cfg.fw, cfg.loss), 0) * d * dh
    if cfg.fw == "linear":
        per_tok = (4 if cfg.loss == "dot" else 6) * d * d
    nm = {"swiglu": 3, "gelu": 2, "linear": 1}[cfg.fw]
    n = d if cfg.fw == "linear" else dh
    ns = cfg.ns_steps * nm * (4.0 * d * d * n + 2.0 * d ** 3)
    P = cfg.batch * cfg.heads
    return P * (cfg.seq_len * per_tok + cfg.n_chunks * ns)


def apply_backward_flops(cfg) -> dict:
    """Algorithmic FLOP of one apply-backward call (one chunk, all problems) per stage: the
    front's Z and dH products, the weight-gradient contractions and dQ."""
    P, b, d, dh = cfg.batch * cfg.heads, cfg.chunk, cfg.dim, cfg.hidden
    nz = {"swiglu": 2, "gelu": 1, "linear": 1}[cfg.fw]
    nm = {"swiglu": 3, "gelu": 2, "linear": 1}[cfg.fw]
    if cfg.fw == "linear":
        return {"contract": 2.0 * b * d * d * P, "dq": 2.0 * b * d * d * P}
    return {"front_k": 2.0 * (nz + 1) * b * d * dh * P, "contract": 2.0 * nm * b * d * dh * P,
            "dq": 2.0 * nz * b * d * dh * P}


def bench_apply_backward(args, cfg, planes):
    """Times ttt_apply_backward on the workload's first chunk (the queries and, as dO, the
    values of that chunk) and prints one JSON line of its own."""
    import numpy as np
    import torch

    import ttt_inputs as ti
    import weight_sequence_layers_amd as W

    c = W.make_config(cfg, planes=planes, path="staged")
    b = cfg.chunk
    P = cfg.batch * cfg.heads
    dev = []
    for name in ("q", "v"):
        blocks = [ti.make_problem_inputs(cfg, bb, h, t1=b) for bb in range(cfg.batch)
                  for h in range(cfg.heads)]
        if cfg.act == "bf16":
            x = np.stack([blk[name + "_bits"] for blk in blocks]).reshape(cfg.batch, cfg.heads, b, -1)
            dev.append(torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16))
        else:
            x = np.stack([blk[name] for blk in blocks]).reshape(cfg.batch, cfg.heads, b, -1)
            dev.append(torch.from_numpy(x).cuda())
    w0 = torch.from_numpy(np.concatenate([w.ravel() for w in ti.make_weights(cfg)])).cuda()
    st = W.ttt_init_state(c, w0)
    dq = torch.empty_like(dev[0])
    dw = torch.empty(W.ttt_state_numel(c), dtype=torch.float32, device="cuda")

    def call():
        W.ttt_apply_backward(st, dev[0], dev[1], dq, dw)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    flops = apply_backward_flops(cfg)
    totals = {}
    for name in flops:
        W.ttt_profile_begin(st, name, 1 << 12)
        call()
        n, ms = W.ttt_profile_end(st)
        if n:
            totals[name] = (n, ms)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    st.destroy()
    total = sum(flops.values())
    print(json.dumps({
        "metric": "apply-step backward tokens/sec (dq and dw of one chunk)",
        "value": round(P * b / dt, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_call": round(1e3 * dt, 3), "higher_is_better": True,
        "dtype": "bf16" if cfg.act == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name} (one chunk of {b} tokens, {P} problems)"},
        "tflops_algorithmic": round(total / dt / 1e12, 2),
        "per_stage_ms": {k: round(v[1], 3) for k, v in totals.items()},
    }), flush=True)


def chunk_backward_flops(cfg) -> dict:
    """Algorithmic FLOP of one ttt_chunk_backward call (one chunk, all problems) per stage, 2
    per multiply-add: the update recomputed (gradient front and contractions, Newton-Schulz
    with its iterates), the Newton-Schulz backward (per iteration A and B' again, then
    T = dX X^T + X dX^T, S = b T + c (T A + A T) and B' dX + S X), the tangent front (six
    products), dK (four), dV (two), the weight contractions (three), and the apply step's
    backward (front, contractions, dQ)."""
    P, b, d, dh = cfg.batch * cfg.heads, cfg.chunk, cfg.dim, cfg.hidden
    m, n, it = d, dh, cfg.ns_steps
    bdh = 2.0 * b * d * dh * P
    f = {
        "front_k": 3 * bdh + 3 * bdh,              # recompute + apply backward's front
        "contract": 3 * bdh + 3 * bdh + 3 * bdh,   # recompute + weight gradients + apply's
        "tfront": 6 * bdh,
        "dq": 4 * bdh + 2 * bdh + 2 * bdh,         # dK, dV, dQ
    }
    if it:
        nm3 = 3 * P * it
        f["ns_gram"] = nm3 * 2.0 * m * m * n * 2   # forward iterates + backward's A
        f["ns_poly"] = nm3 * 2.0 * m ** 3 * 2
        f["ns_update"] = nm3 * 2.0 * m * m * n
        f["ns_bwd"] = nm3 * (2 * 2.0 * m * m * n + 2 * 2.0 * m ** 3 + 2 * 2.0 * m * m * n)
    return f


def bench_chunk_backward(args, cfg, planes):
    """Times ttt_chunk_backward on the workload's first chunk (state W0, cotangents drawn
    from a seeded normal) and prints one JSON line of its own."""
    import numpy as np
    import torch

    import ttt_inputs as ti
    import weight_sequence_layers_amd as W

    c = W.make_config(cfg, planes=planes, path="staged")
    b = cfg.chunk
    P = cfg.batch * cfg.heads
    blocks = [ti.make_problem_inputs(cfg, bb, h, t1=b) for bb in range(cfg.batch)
              for h in range(cfg.heads)]
    dev = {}
    for name in ("q", "k", "v"):
        if cfg.act == "bf16":
            x = np.stack([blk[name + "_bits"] for blk in blocks]).reshape(cfg.batch, cfg.heads, b, -1)
            dev[name] = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
        else:
            x = np.stack([blk[name] for blk in blocks]).reshape(cfg.batch, cfg.heads, b, -1)
            dev[name] = torch.from_numpy(x).cuda()
    eta = torch.from_numpy(np.stack([blk["eta"] for blk in blocks]).reshape(
        cfg.batch, cfg.heads, b)).cuda()
    g = torch.Generator(device="cuda").manual_seed(7)
    dout = torch.randn(dev["q"].shape, generator=g, device="cuda").to(dev["q"].dtype)
    w0 = torch.from_numpy(np.concatenate([w.ravel() for w in ti.make_weights(cfg)])).cuda()
    st = W.ttt_init_state(c, w0)
    n = W.ttt_state_numel(c)
    dw_in = torch.randn(n, generator=g, device="cuda")
    dw = torch.empty_like(dw_in)
    grads = [torch.empty_like(dev["q"]) for _ in range(3)]
    deta = torch.empty_like(eta)

    def call():
        dw.copy_(dw_in)
        W.ttt_chunk_backward(st, dev["q"], dev["k"], dev["v"], eta, dout, dw, *grads, deta)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    flops = chunk_backward_flops(cfg)
    totals = {}
    for name in flops:
        W.ttt_profile_begin(st, name, 1 << 12)
        call()
        k, ms = W.ttt_profile_end(st)
        if k:
            totals[name] = (k, ms)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    W.ttt_state_health(st)
    st.destroy()
    total = sum(flops.values())
    dom = max(totals, key=lambda x: totals[x][1])
    per_launch = flops[dom] / totals[dom][0]
    achieved = per_launch / (totals[dom][1] / totals[dom][0] / 1e3) / 1e12
    print(json.dumps({
        "metric": "chunk backward tokens/sec (dq, dk, dv, deta and the state cotangent)",
        "value": round(P * b / dt, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_call": round(1e3 * dt, 3), "higher_is_better": True,
        "dtype": "bf16" if cfg.act == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name} (one chunk of {b} tokens, {P} problems)",
                   "bf16_planes_apply_grad_ns": list(planes[:3]),
                   "ns_one_plane_iterations": [i for i in range(8) if (planes[3] >> i) & 1],
                   **({"momentum": cfg.momentum} if cfg.momentum else {})},
        "tflops_algorithmic": round(total / dt / 1e12, 2),
        "pct_bf16_peak_algorithmic": round(100 * total / dt / 1e12 / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "kernel": dom},
        "per_stage_ms": {k: round(v[1], 3) for k, v in totals.items()},
    }), flush=True)


# The LaCT block around each workload's TTT layer: model width = heads x dim, attention
# heads of 128, the window of the page's reading (text: a sliding window of one chunk;
# image sets: one image of 8040 tokens, 1,029,120 / 128), MLP hidden 4 x width.
BLOCK_WINDOW = {"lm": (2048, "sliding"), "long": (4096, "sliding"),
                "imageset": (8040, "block"), "smallchunk": (64, "sliding")}


def block_part_flops(cfg, dim: int, F: int, window: int, mode: str) -> dict:
    """Algorithmic FLOP per step of each part of the block (2 per multiply-add): the
    projections, the attention (4 x 128 per head and allowed (query, key) pair) and the
    TTT layer (total_flops)."""
    B, T, H = cfg.batch, cfg.seq_len, cfg.heads
    rows = B * T
    if mode == "sliding":
        pairs = sum(min(t + 1, window) for t in range(T)) if T <= 1 << 20 else T * window
    else:
        full, rest = divmod(T, window)
        pairs = full * window * window + rest * rest
    return {"proj_qkv": 2 * 2.0 * rows * dim * 3 * dim,      # attention and TTT q, k, v
            "proj_out": 2 * 2.0 * rows * dim * dim,          # attention and TTT outputs
            "ffn_up": 2.0 * rows * dim * F, "ffn_down": 2.0 * rows * F * dim,
            "attention": 4.0 * 128 * pairs * B * (dim // 128),
            "ttt_layer": total_flops(cfg)}


def bench_block(args, cfg, planes):
    """Times ttt_block_forward over the workload's whole batch (one step = one block over
    every sequence) and each of its parts on its own, and prints one JSON line."""
    import numpy as np
    import torch

    import oracle.ttt_block as blk_oracle
    import ttt_inputs as ti
    import weight_sequence_layers_amd as W

    if cfg.name not in BLOCK_WINDOW:
        sys.exit(f"no block shape for workload {cfg.name}")
    window, mode = BLOCK_WINDOW[cfg.name]
    D = cfg.heads * cfg.dim
    F = 4 * D
    B, T = cfg.batch, cfg.seq_len
    c = W.make_config(cfg, planes=planes)
    bc = W.make_block_config(c, dim=D, window=window, mode=mode, ffn_hidden=F, max_seq_len=T)
    t = time.perf_counter()
    inp = ti.make_block_inputs(B, T, D, F, cfg.heads, cfg.seed)
    log(f"block inputs generated in {time.perf_counter() - t:.1f} s")

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)

    weights = {n: dev(inp[n + "_bits"]) for n in ti.BLOCK_WEIGHT_NAMES}
    x = dev(inp["x_bits"])
    y = torch.empty_like(x)
    w0list = ti.make_weights(cfg)
    w0 = torch.from_numpy(np.concatenate([w.ravel() for w in w0list])).cuda()
    blk = W.ttt_block_init(bc, weights, w0)

    def step():
        W.ttt_block_forward(blk, x, y, T)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    W.ttt_state_health(W.ttt_block_ttt_state(blk))

    # each part on its own, with HIP events on the current stream (torch's, which the
    # calls launch on)
    rows = B * T
    g = torch.Generator(device="cuda").manual_seed(3)
    qkv = torch.randn(rows, 3 * D, generator=g, device="cuda").to(torch.bfloat16)
    a_out = torch.empty(rows, D, dtype=torch.bfloat16, device="cuda")
    h = torch.empty(rows, F, dtype=torch.bfloat16, device="cuda")

    def timed(fn, reps=max(args.steps, 3)):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    xr = x.view(rows, D)
    parts = {
        "attention": (1, timed(lambda: W.ttt_window_attention(
            qkv, qkv[:, D:], qkv[:, 2 * D:], 3 * D, a_out, D, B, D // 128, T, window, mode))),
        "proj_qkv": (2, timed(lambda: W.ttt_linear(xr, weights["attn_qkv"], None, qkv, rows,
                                                   D, 3 * D, "plain"))),
        "proj_out": (2, timed(lambda: W.ttt_linear(xr, weights["attn_out"], a_out, a_out, rows,
                                                   D, D, "residual"))),
        "ffn_up": (1, timed(lambda: W.ttt_linear(xr, weights["ffn_up"], None, h, rows, D, F,
                                                 "gelu"))),
        "ffn_down": (1, timed(lambda: W.ttt_linear(h, weights["ffn_down"], a_out, a_out, rows,
                                                   F, D, "residual"))),
    }
    del qkv, h
    tin = ti.make_inputs(cfg)
    tdev = [torch.from_numpy(tin[n + "_bits"].view(np.int16)).cuda().view(torch.bfloat16)
            for n in ("q", "k", "v")]
    teta = torch.from_numpy(tin["eta"]).cuda()
    tout = torch.empty_like(tdev[0])
    del tin
    st = W.ttt_init_state(c, w0)
    parts["ttt_layer"] = (1, timed(lambda: W.ttt_sequence_forward(st, *tdev, teta, tout, T)))
    st.destroy()
    del tdev, tout
    flops = block_part_flops(cfg, D, F, window, mode)
    own = {k: v for k, v in parts.items() if k != "ttt_layer"}
    dom = max(own, key=lambda k: own[k][0] * own[k][1])
    per_launch = flops[dom] / parts[dom][0]
    achieved = per_launch / (parts[dom][1] / 1e3) / 1e12
    total = sum(flops.values())

    # the oracle: one sequence's first four chunks (or the first 8192 tokens of one image
    # set), the same weights and initial fast weights
    Tc = min(T, 4 * cfg.chunk if cfg.chunk < T else 8192)
    cpu = None
    if not args.no_cpu_baseline and (cfg.order == "apply_then_update" or Tc == T):
        class BC:
            pass
        bco = BC()
        bco.ttt = cfg.replace(seq_len=Tc, batch=1)
        bco.window, bco.window_mode = window, mode
        per_head = [[w[hh] for w in w0list] for hh in range(cfg.heads)]
        t1 = time.perf_counter()
        blk_oracle.block_forward(bco, inp, inp["x"][0, :Tc].astype(np.float64), per_head)
        odt = time.perf_counter() - t1
        cpu = {"value": Tc / odt, "unit": "tokens/s", "cores": os.cpu_count(), "kind": "oracle",
               "sample": f"one sequence's first {Tc} tokens through the block oracle "
                         f"(numpy fp64), {odt:.1f} s"}
    blk.destroy()
    res = {
        "metric": "LaCT block tokens/sec (window attention + TTT layer + MLP)",
        "value": round(B * T / dt, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(1e3 * dt, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name} block: batch {B}, seq {T}, width {D} "
                               f"({D // 128} attention heads, {cfg.heads} TTT heads of "
                               f"{cfg.dim}), {mode} window {window}, MLP {F}, TTT chunk "
                               f"{cfg.chunk}",
                   "bf16_planes_apply_grad_ns": list(planes[:3])},
        "block_tflops_algorithmic": round(total / dt / 1e12, 2),
        "parts_ms_per_step": {k: round(n * ms, 3) for k, (n, ms) in parts.items()},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": dom,
                     "avg_launch_us": round(1e3 * parts[dom][1], 2)},
        "parts_tflops": {k: round(flops[k] / (n * ms / 1e3) / 1e12, 1)
                         for k, (n, ms) in parts.items()},
    }
    if cpu:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


def traffic_for(args, workload: str, stage: str):
    """recorded_traffic for a run of the workload as profiled; None when the command line
    changes its kernels' work (batch, momentum, step sizes, decay, planes)."""
    if args.batch or args.momentum or args.lr or args.weight_decay or args.planes:
        return None
    return recorded_traffic(workload, stage)


def recorded_traffic(workload: str, stage: str):
    """HBM bytes per launch of `stage` from profiles/<workload>_traffic.md, if that summary
    was taken from the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    digest, val = None, None
    for line in open(path):
        if line.startswith("source digest:"):
            digest = line.split(":", 1)[1].strip()
        if line.startswith(f"| {stage} |"):
            val = float(line.split("|")[-2])
    from weight_sequence_layers_amd.profiling import source_digest
    return val if digest == source_digest() else None


def blas_reference(cfg, planes, reps: int = 10) -> dict:
    """hipBLASLt (torch.bmm, bf16) on the GEMM shapes of each stage, with the K dimension
    multiplied by the plane products the stage executes; context for the stage kernels'
    rates (no epilogues, no symmetry savings, no fusion)."""
    import torch
    P, b, d, dh = cfg.batch * cfg.heads, cfg.chunk, cfg.dim, cfg.hidden
    nm = {"swiglu": 3, "gelu": 2, "linear": 1}[cfg.fw]
    nz = {"swiglu": 2, "gelu": 1, "linear": 1}[cfg.fw]
    n = d if cfg.fw == "linear" else dh
    ap, gp, npl = planes[0], planes[1], planes[2]
    ns_prod = npl * (npl + 1) // 2
    b = min(b, 8192)
    shapes = {}
    if cfg.fw != "linear":
        shapes["front_q"] = (P * nz, b, dh, d * ap)
        shapes["front_k"] = (P * (nz + (cfg.loss == "dot")), b, dh, d * gp)
        shapes["out"] = (P, b, d, dh * ap)
    shapes["contract"] = (P * nm, d, n, b * gp)
    if cfg.ns_steps:
        shapes["ns_gram"] = (P * nm, d, d, n * ns_prod)
        shapes["ns_poly"] = (P * nm, d, d, d * ns_prod)
        shapes["ns_update"] = (P * nm, d, n, d * ns_prod)
    out = {}
    for name, (B, M, N, K) in shapes.items():
        x = torch.randn(B, M, K, device="cuda", dtype=torch.bfloat16)
        y = torch.randn(B, K, N, device="cuda", dtype=torch.bfloat16)
        for _ in range(2):
            torch.bmm(x, y)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.bmm(x, y)
        e1.record()
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / reps
        tf = 2.0 * B * M * N * K / us / 1e6
        out[name] = {"bmm": [B, M, N, K], "us": round(us, 1), "tflops": round(tf, 1),
                     "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 3)}
        del x, y
    return out


def cpu_baseline(cfg, budget_chunks=None, min_seconds=10.0):
    """The oracle on the host: (batch, head) problems in order, each over its first
    chunks, until min_seconds of oracle time have been spent or every problem is done."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle.ttt_oracle as orc
    import ttt_inputs as ti

    nc = cfg.n_chunks if budget_chunks is None else min(cfg.n_chunks, budget_chunks)
    T = nc * cfg.chunk
    weights = ti.make_weights(cfg)
    problems = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    dt, done = 0.0, 0
    for (b, h) in problems:
        p = ti.make_problem_inputs(cfg, b, h, t1=T)
        w0 = [w[h] for w in weights]
        t0 = time.perf_counter()
        orc.sequence_forward(cfg, w0, p["q"], p["k"], p["v"], p["eta"], n_chunks=nc)
        dt += time.perf_counter() - t0
        done += 1
        if dt >= min_seconds:
            break
    T *= done
    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("internal_api") in ("openblas", "mkl", "blis")] or [1])
    model = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {len(problems)} (batch, head) problems, {nc} chunks each "
                      f"({T} tokens), numpy fp64, {dt:.1f} s on {model}; problems are "
                      f"independent so the rate is the whole workload's"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="lm")
    ap.add_argument("--planes", default=None, help="apply,grad,ns bf16 plane counts and the ns_one_plane iteration mask")
    ap.add_argument("--lr", default=None,
                    help="comma-separated step sizes per matrix (state order); default 1")
    ap.add_argument("--weight-decay", type=float, default=0.0)
    ap.add_argument("--batch", type=int, default=None,
                    help="another batch size than the workload's (more problems per launch)")
    ap.add_argument("--momentum", type=float, default=0.0,
                    help="heavy-ball coefficient over chunk gradients (the workload's is 0)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--apply-backward", action="store_true",
                    help="time the apply-step backward on the workload's first chunk instead")
    ap.add_argument("--replay", action="store_true",
                    help="record each step's launches in a HIP graph and replay it")
    ap.add_argument("--chunk-backward", action="store_true",
                    help="time the backward through one chunk on the workload's first chunk")
    ap.add_argument("--block", action="store_true",
                    help="time the LaCT block around the workload's layer instead")
    ap.add_argument("--cpu-chunks", type=int, default=None)
    ap.add_argument("--blas-reference", action="store_true",
                    help="also time hipBLASLt (torch.bmm) on each stage's GEMM shapes")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before the steps, run one plain device copy of this many MiB (a "
                         "known-size reference for rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the layer's (batch, head) problems shard across GPUs with no communication, "
              "and this benchmark measures one GPU's throughput)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import ttt_inputs as ti
    import weight_sequence_layers_amd as W
    from weight_sequence_layers_amd.profiling import source_digest

    cfg = ti.CONFIGS[args.workload]
    if args.lr or args.weight_decay:
        cfg = cfg.replace(lr=tuple(float(x) for x in (args.lr or "").split(",") if x),
                          weight_decay=args.weight_decay)
    if args.momentum:
        cfg = cfg.replace(momentum=args.momentum)
    if args.batch:
        cfg = cfg.replace(batch=args.batch)
    planes = tuple(int(x) for x in args.planes.split(",")) if args.planes else W.PRECISION[cfg.name]
    if args.apply_backward:
        bench_apply_backward(args, cfg, planes)
        return
    if args.chunk_backward:
        bench_chunk_backward(args, cfg, planes)
        return
    if args.block:
        bench_block(args, cfg, planes)
        return
    c = W.make_config(cfg, planes=planes, replay=args.replay)
    torch.cuda.set_device(0)
    log(f"workload {cfg}  planes {planes}")

    t = time.perf_counter()
    inp = ti.make_inputs(cfg)
    log(f"inputs generated in {time.perf_counter() - t:.1f} s")
    dev = []
    for n in ("q", "k", "v"):
        if cfg.act == "bf16":
            dev.append(torch.from_numpy(inp[n + "_bits"].view(np.int16)).cuda().view(torch.bfloat16))
        else:
            dev.append(torch.from_numpy(inp[n]).cuda())
    eta = torch.from_numpy(inp["eta"]).cuda()
    w0 = torch.from_numpy(np.concatenate([w.ravel() for w in inp["w0"]])).cuda()
    out = torch.empty_like(dev[0])
    del inp
    st = W.ttt_init_state(c, w0)
    if args.calib_copy_mib:
        # one elementwise kernel that reads and writes exactly this many bytes each
        n = (args.calib_copy_mib << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.add(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    def step():
        W.ttt_sequence_forward(st, *dev, eta, out, cfg.seq_len)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # find the stage with the largest total time (one traced step per stage, untimed)
    flops = stage_flops(cfg)
    totals = {}
    for name in flops:
        W.ttt_profile_begin(st, name, 1 << 14)
        step()
        n, ms = W.ttt_profile_end(st)
        if n:
            totals[name] = (n, ms)
    dom = max(totals, key=lambda k: totals[k][1])
    log("per-stage time in one step: " + ", ".join(
        f"{k} {v[1]:.3f} ms/{v[0]}" for k, v in sorted(totals.items(), key=lambda x: -x[1][1])))

    # timed region: plain steps, no events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # the same number of steps again with the dominant stage's launches bracketed by HIP
    # events on the launch stream (the events' own cost stays out of the headline)
    W.ttt_profile_begin(st, dom, 1 << 16)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    n_dom, ms_dom = W.ttt_profile_end(st)
    W.ttt_state_health(st)
    log(f"ms per step: {1e3 * (t1 - t0) / args.steps:.3f} plain, "
        f"{1e3 * (t3 - t2) / args.steps:.3f} with the {dom} events")

    elapsed = t1 - t0
    ms_per_step = 1e3 * elapsed / args.steps
    tokens = cfg.batch * cfg.seq_len
    value = tokens * args.steps / elapsed
    tf_layer = total_flops(cfg) / (elapsed / args.steps) / 1e12
    avg_s = ms_dom / max(n_dom, 1) / 1e3
    # algorithmic FLOP of one launch: the stage's FLOP per step over its launches per step
    per_launch = flops[dom] / (n_dom / args.steps)
    achieved = per_launch / avg_s / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_for(args, cfg.name, dom), "kernel": dom,
                "avg_launch_us": round(avg_s * 1e6, 2),
                "launches": n_dom}
    res = {
        "metric": "TTT-layer tokens/sec (update+apply) at chunk 2048; % bf16 MFMA peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: batch {cfg.batch}, heads {cfg.heads}, seq "
                               f"{cfg.seq_len}, chunk {cfg.chunk}, dim {cfg.dim}, hidden "
                               f"{cfg.hidden}, {cfg.fw}/{cfg.loss}, ns {cfg.ns_steps}, renorm "
                               f"{int(cfg.renorm)}, {cfg.act}, {cfg.order}",
                   "global_batch": cfg.batch, "seq_len": cfg.seq_len, "parallelism": "none",
                   "bf16_planes_apply_grad_ns": list(planes[:3]), "ns_one_plane_iterations": [i for i in range(8) if (planes[3] >> i) & 1],
                   "replay": bool(args.replay),
                   **({"lr": list(cfg.step_sizes()), "weight_decay": cfg.weight_decay}
                      if (cfg.lr or cfg.weight_decay) else {}),
                   **({"momentum": cfg.momentum} if cfg.momentum else {})},
        "source_digest": source_digest(),
        "layer_tflops_algorithmic": round(tf_layer, 2),
        "pct_bf16_peak_algorithmic": round(100 * tf_layer / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline,
    }
    st.destroy()
    if args.blas_reference:
        res["blas_reference"] = blas_reference(cfg, planes)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, args.cpu_chunks)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
