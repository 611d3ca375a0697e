"""GPU parity of the LaCT block calls (include/ttt_block.h) against the block oracle
(oracle/ttt_block.py) on seeded inputs.

Bars:
bf16 keeps 8 significant bits, so one rounding to nearest moves a value by at most half an
ulp, 2^-8 of its magnitude.
* window attention, element by element: |o - o_ref| <= 2^-8 |o_ref| + 2^-7 max|v| + 1e-6.
  The output is rounded once to bf16; the probabilities are rounded to bf16 (2^-8 relative
  each) and the normaliser sums the rounded values, so the output is the exact average
  under weights each within 2^-8 of the true ones, which moves it by at most
  2^-8 max_j |v_j - o| <= 2^-7 max|v|; fp32 scores and sums add ~1e-6.
* projections, element by element: |y - y_ref| <= 2^-8 |y_ref| + 2^-16 sum_i |x_i w_i| + 1e-6
  (one bf16 rounding of the fp32 result; fp32 accumulation of the products well inside
  2^-16 of their absolute sum at these lengths; the GELU and the residual add are fp32).
* the whole block: max relative error per tensor (|y - y_ref|_inf / |y_ref|_inf) <= 2e-2 on
  y and on every final fast-weight matrix, the bf16 bar of the TTT layer's own parity (the
  layer sits inside the block; the storage roundings the block adds are each at most
  2^-8 of values of the output's scale).
"""
import numpy as np
import pytest
import torch

import oracle.ttt_block as blk
import oracle.ttt_oracle as orc
import ttt_inputs as ti
import weight_sequence_layers_amd as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def _bits(x):
    return ti.bf16_round(np.asarray(x, np.float32))


# ------------------------------------------------------------------------ window attention
def _attention_case(B, heads, T, window, mode, seed, qscale=1.0):
    rng = np.random.default_rng(seed)
    D = heads * 128
    qkv = rng.standard_normal((B, T, 3 * D)).astype(np.float32)
    qkv[..., :D] *= qscale
    vals, bits = _bits(qkv)
    dev = _bf16_dev(bits)
    out = torch.zeros(B, T, D, dtype=torch.bfloat16, device=DEV)
    print(f"attention B={B} heads={heads} T={T} window={window} {mode}", flush=True)
    W.ttt_window_attention(dev, dev[..., D:], dev[..., 2 * D:], 3 * D, out, D, B, heads, T,
                           window, mode)
    torch.cuda.synchronize()
    return vals.astype(np.float64), out.float().cpu().numpy().astype(np.float64)


def _attention_bar(o_ref, vmax):
    return 2.0 ** -8 * np.abs(o_ref) + 2.0 ** -7 * vmax + 1e-6


@pytest.mark.parametrize("B,heads,T,window,mode,qscale", [
    (2, 2, 300, 37, "sliding", 1.0),
    (1, 1, 300, 1, "sliding", 1.0),
    (1, 2, 300, 64, "sliding", 1.0),
    (2, 1, 300, 128, "sliding", 4.0),
    (1, 1, 300, 1000, "sliding", 1.0),
    (1, 3, 257, 200, "sliding", 8.0),
    (2, 2, 300, 50, "block", 1.0),
    (1, 1, 300, 64, "block", 4.0),
    (1, 2, 300, 300, "block", 1.0),
    (1, 1, 1, 5, "sliding", 1.0),
    (1, 1, 1, 5, "block", 1.0),
])
def test_window_attention_matches_oracle(B, heads, T, window, mode, qscale):
    qkv, got = _attention_case(B, heads, T, window, mode, 11 + T + window, qscale)
    D = heads * 128
    worst = 0.0
    for b in range(B):
        for h in range(heads):
            s = slice(h * 128, (h + 1) * 128)
            q, k, v = qkv[b, :, s], qkv[b, :, D:][:, s], qkv[b, :, 2 * D:][:, s]
            ref = blk.window_attention(q, k, v, window, mode)
            err = np.abs(got[b, :, s] - ref)
            bar = _attention_bar(ref, np.abs(v).max())
            assert np.all(err <= bar), (b, h, float((err - bar).max()))
            worst = max(worst, float((err / bar).max()))
    print(f"  worst error / bar {worst:.3f}", flush=True)


@pytest.mark.parametrize("window", [777, 64])
def test_window_attention_many_workgroups(window):
    """A launch of a thousand workgroups: 4 sequences x 8 heads x 4000 tokens (a ragged last
    workgroup per head), whole heads compared."""
    B, heads, T = 4, 8, 4000
    qkv, got = _attention_case(B, heads, T, window, "sliding", 31 + window)
    D = heads * 128
    for b, h in ((0, 0), (3, 7), (2, 5)):
        s = slice(h * 128, (h + 1) * 128)
        q, k, v = qkv[b, :, s], qkv[b, :, D:][:, s], qkv[b, :, 2 * D:][:, s]
        ref = blk.window_attention(q, k, v, window, "sliding")
        err = np.abs(got[b, :, s] - ref)
        bar = _attention_bar(ref, np.abs(v).max())
        assert np.all(err <= bar), (b, h, float((err - bar).max()))


def test_window_attention_empty_sequence_writes_nothing():
    out = torch.full((1, 4, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    x = torch.zeros(1, 4, 3 * 128, dtype=torch.bfloat16, device=DEV)
    W.ttt_window_attention(x, x[..., 128:], x[..., 256:], 384, out, 128, 1, 1, 0, 8, "sliding")
    torch.cuda.synchronize()
    assert bool((out == 7).all())


@pytest.mark.parametrize("mode,window", [("sliding", 2048), ("block", 8040)])
def test_window_attention_full_size_sampled(mode, window):
    """The language-model block's attention shape (4 x 32768 tokens, 8 heads, window 2048)
    and the image-set shape's window (8040 tokens per image), checked on sampled queries
    that the oracle computes one by one over their own windows."""
    B, heads, T = (4, 8, 32768) if mode == "sliding" else (1, 2, 3 * 8040 + 77)
    D = heads * 128
    g = torch.Generator(device=DEV).manual_seed(5)
    qkv = torch.randn(B, T, 3 * D, generator=g, device=DEV).to(torch.bfloat16)
    out = torch.empty(B, T, D, dtype=torch.bfloat16, device=DEV)
    print(f"attention full size B={B} heads={heads} T={T} window={window} {mode}", flush=True)
    W.ttt_window_attention(qkv, qkv[..., D:], qkv[..., 2 * D:], 3 * D, out, D, B, heads, T,
                           window, mode)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    ts = sorted(set([0, 1, 63, 64, 127, 128, window - 1, window, window + 1, T - 1, T - 2] +
                    list(rng.integers(0, T, 40))))
    ts = [t for t in ts if 0 <= t < T]
    for b in {0, B - 1}:
        for h in {0, heads - 1}:
            s = slice(h * 128, (h + 1) * 128)
            for t in ts:
                if mode == "sliding":
                    lo, hi = max(0, t - window + 1), t + 1
                else:
                    lo = t // window * window
                    hi = min(T, lo + window)
                rows = qkv[b, lo:hi].float().cpu().numpy().astype(np.float64)
                q = qkv[b, t, s].float().cpu().numpy().astype(np.float64)
                k, v = rows[:, D:][:, s], rows[:, 2 * D:][:, s]
                sc = k @ q / np.sqrt(128.0)
                p = np.exp(sc - sc.max())
                ref = p @ v / p.sum()
                got = out[b, t, s].float().cpu().numpy()
                bar = _attention_bar(ref, np.abs(v).max())
                assert np.all(np.abs(got - ref) <= bar), (b, h, t)


# ------------------------------------------------------------------------ projections
@pytest.mark.parametrize("epi", ["plain", "residual", "gelu"])
@pytest.mark.parametrize("rows,K,N", [(300, 256, 384), (1, 8, 8), (129, 1000, 136)])
def test_linear_matches_definition(epi, rows, K, N):
    rng = np.random.default_rng(rows + K + N)
    xv, xb = _bits(rng.standard_normal((rows, K)))
    wv, wb = _bits(rng.standard_normal((N, K)) / np.sqrt(K))
    rv, rb = _bits(rng.standard_normal((rows, N)))
    x, w, r = _bf16_dev(xb), _bf16_dev(wb), _bf16_dev(rb)
    y = torch.empty(rows, N, dtype=torch.bfloat16, device=DEV)
    print(f"linear {epi} rows={rows} K={K} N={N}", flush=True)
    W.ttt_linear(x, w, r if epi == "residual" else None, y, rows, K, N, epi)
    torch.cuda.synchronize()
    X, Wt = xv.astype(np.float64), wv.astype(np.float64)
    acc = X @ Wt.T
    ref = {"plain": acc, "residual": rv.astype(np.float64) + acc, "gelu": blk.gelu(acc)}[epi]
    bar = 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * (np.abs(X) @ np.abs(Wt).T) + 1e-6
    err = np.abs(y.float().cpu().numpy() - ref)
    assert np.all(err <= bar), float((err - bar).max())


# 8200 x 4104 outputs at 2056 input features give 561 tiles of 256 x 256 and a long K loop,
# so those launches take the wide-tile kernel, with ragged rows, output features and a
# partial last K step
WIDE = (8200, 2056, 4104)


@pytest.mark.parametrize("epi", ["plain", "residual", "gelu"])
def test_linear_wide_tiles_sampled(epi):
    rows, K, N = WIDE
    rng = np.random.default_rng(17)
    xv, xb = _bits(rng.standard_normal((rows, K)))
    wv, wb = _bits(rng.standard_normal((N, K)) / np.sqrt(K))
    rv, rb = _bits(rng.standard_normal((rows, N)))
    x, w, r = _bf16_dev(xb), _bf16_dev(wb), _bf16_dev(rb)
    y = torch.empty(rows, N, dtype=torch.bfloat16, device=DEV)
    print(f"linear wide {epi} rows={rows} K={K} N={N}", flush=True)
    W.ttt_linear(x, w, r if epi == "residual" else None, y, rows, K, N, epi)
    torch.cuda.synchronize()
    # rows from every 256-row tile at several offsets, and the ragged last tile
    sel = np.unique(np.concatenate([np.arange(0, rows, 97), np.arange(rows - 8, rows)]))
    X, Wt = xv[sel].astype(np.float64), wv.astype(np.float64)
    acc = X @ Wt.T
    ref = {"plain": acc, "residual": rv[sel].astype(np.float64) + acc, "gelu": blk.gelu(acc)}[epi]
    bar = 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * (np.abs(X) @ np.abs(Wt).T) + 1e-6
    err = np.abs(y.float().cpu().numpy()[sel] - ref)
    assert np.all(err <= bar), float((err - bar).max())


@pytest.mark.parametrize("rows,K,N", [(200, 128, 256), WIDE])
def test_linear_residual_in_place(rows, K, N):
    rng = np.random.default_rng(9)
    xv, xb = _bits(rng.standard_normal((rows, K)))
    wv, wb = _bits(rng.standard_normal((N, K)) / np.sqrt(K))
    rv, rb = _bits(rng.standard_normal((rows, N)))
    x, w, r = _bf16_dev(xb), _bf16_dev(wb), _bf16_dev(rb)
    y = torch.empty_like(r)
    print(f"linear in place rows={rows} K={K} N={N}", flush=True)
    W.ttt_linear(x, w, r, y, rows, K, N, "residual")
    W.ttt_linear(x, w, r, r, rows, K, N, "residual")
    torch.cuda.synchronize()
    assert torch.equal(y, r)


# ------------------------------------------------------------------------ the block
def _block_case(B, T, dim, ttt_heads, chunk, window, mode, order, seed, ffn=0):
    d = dim // ttt_heads
    tcfg = ti.Config("block", B, ttt_heads, T, chunk, d, 2 * d, "swiglu", "dot", 5, True,
                     "bf16", order, seed)
    F = ffn or 4 * dim
    inp = ti.make_block_inputs(B, T, dim, F, ttt_heads, seed)
    w0 = ti.make_weights(tcfg)

    class BC:
        pass
    bc = BC()
    bc.ttt, bc.window, bc.window_mode = tcfg, window, mode
    return tcfg, F, inp, w0, bc


def _run_block(tcfg, F, inp, w0, dim, window, mode, T, max_T=None, calls=1):
    c = W.make_config(tcfg)
    bcfg = W.make_block_config(c, dim=dim, window=window, mode=mode, ffn_hidden=F,
                               max_seq_len=max_T or T)
    weights = {n: _bf16_dev(inp[n + "_bits"]) for n in ti.BLOCK_WEIGHT_NAMES}
    w0d = torch.from_numpy(np.concatenate([w.ravel() for w in w0])).to(DEV)
    blkh = W.ttt_block_init(bcfg, weights, w0d)
    x = _bf16_dev(inp["x_bits"])
    y = torch.empty_like(x)
    for _ in range(calls):
        W.ttt_block_forward(blkh, x, y, T)
    st = W.ttt_block_ttt_state(blkh)
    flat = torch.empty(W.ttt_state_numel(c), dtype=torch.float32, device=DEV)
    W.ttt_get_state(st, flat)
    torch.cuda.synchronize()
    Ws = [m.cpu().numpy().astype(np.float64) for m in W.split_state(c, flat)]
    W.ttt_block_destroy(blkh)
    return y.float().cpu().numpy().astype(np.float64), Ws


def _rel(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))


@pytest.mark.parametrize("B,T,dim,heads,chunk,window,mode,order", [
    (2, 192, 256, 2, 64, 48, "sliding", "apply_then_update"),
    (1, 256, 256, 1, 128, 100, "sliding", "apply_then_update"),
    (1, 200, 384, 3, 200, 50, "block", "update_then_apply"),
    (1, 256, 768, 1, 256, 100, "block", "update_then_apply"),
])
def test_block_matches_oracle(B, T, dim, heads, chunk, window, mode, order):
    tcfg, F, inp, w0, bc = _block_case(B, T, dim, heads, chunk, window, mode, order, 77 + T)
    print(f"block B={B} T={T} D={dim} ttt heads={heads} chunk={chunk} window={window} {mode}",
          flush=True)
    y, Ws = _run_block(tcfg, F, inp, w0, dim, window, mode, T, max_T=T + chunk, calls=2)
    worst_y, worst_w = 0.0, 0.0
    for b in range(B):
        per_head = [[w[h] for w in w0] for h in range(heads)]
        y_ref, states = blk.block_forward(bc, inp, inp["x"][b].astype(np.float64), per_head,
                                          return_states=True)
        worst_y = max(worst_y, _rel(y[b], y_ref))
        for h in range(heads):
            for m, Wm in enumerate(states[h]):
                worst_w = max(worst_w, _rel(Ws[m][b, h], Wm))
    print(f"  y {worst_y:.3e}  W {worst_w:.3e}", flush=True)
    assert worst_y <= 2e-2 and worst_w <= 2e-2, (worst_y, worst_w)


def test_block_empty_and_rejected_lengths():
    tcfg, F, inp, w0, bc = _block_case(1, 128, 256, 2, 64, 32, "sliding", "apply_then_update", 3)
    c = W.make_config(tcfg)
    bcfg = W.make_block_config(c, dim=256, window=32, mode="sliding", ffn_hidden=F,
                               max_seq_len=128)
    weights = {n: _bf16_dev(inp[n + "_bits"]) for n in ti.BLOCK_WEIGHT_NAMES}
    w0d = torch.from_numpy(np.concatenate([w.ravel() for w in w0])).to(DEV)
    blkh = W.ttt_block_init(bcfg, weights, w0d)
    x = _bf16_dev(inp["x_bits"])
    y = torch.full_like(x, 3.0)
    W.ttt_block_forward(blkh, x, y, 0)
    torch.cuda.synchronize()
    assert bool((y == 3).all())
    for bad in (100, 192):   # not a multiple of the chunk; beyond max_seq_len
        with pytest.raises(W.TTTError):
            W.ttt_block_forward(blkh, x, y, bad)
    W.ttt_block_destroy(blkh)


def test_block_full_size_first_chunk():
    """The LaCT language-model block at the benchmark's shape (4 sequences of 32768 tokens,
    width 1024, TTT heads 2 x 512, chunk 2048, sliding window 2048, MLP 4096) through the same
    call the benchmark times. Under the shifted order the first chunk's queries see the
    initial fast weights and the window is causal, so rows t < 2048 depend on x[0..2047]
    alone: the oracle computes them from a 2048-token sequence, for the first and last
    sequence of the batch."""
    cfg = ti.CONFIGS["lm"]
    B, T, D, F, H = cfg.batch, cfg.seq_len, cfg.heads * cfg.dim, 4 * cfg.heads * cfg.dim, cfg.heads
    inp = ti.make_block_inputs(B, T, D, F, H, cfg.seed)
    w0 = ti.make_weights(cfg)
    print(f"block full size B={B} T={T} D={D}", flush=True)
    y, _ = _run_block(cfg, F, inp, w0, D, cfg.chunk, "sliding", T)
    b0 = cfg.chunk

    class BC:
        pass
    bc = BC()
    bc.ttt, bc.window, bc.window_mode = cfg.replace(seq_len=b0, batch=1), cfg.chunk, "sliding"
    per_head = [[w[h] for w in w0] for h in range(H)]
    for b in (0, B - 1):
        y_ref = blk.block_forward(bc, inp, inp["x"][b, :b0].astype(np.float64), per_head)
        err = _rel(y[b, :b0], y_ref)
        print(f"  sequence {b}: first chunk max rel err {err:.3e}", flush=True)
        assert err <= 2e-2, (b, err)
    assert np.isfinite(y).all()
