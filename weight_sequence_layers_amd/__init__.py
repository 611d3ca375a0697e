"""Python binding of libttt, the large-chunk TTT layer forward for MI355X (gfx950).

Argument marshalling only: every step of the layer runs in the HIP kernels of libttt.so.
PyTorch supplies device memory and the current stream. The functions carry the C names
(ttt_init_state, ttt_chunk_forward, ttt_sequence_forward, ...) and raise TTTError on any
non-OK status. If libttt.so is missing or cannot be loaded, every call raises: there is
no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
# LIBTTT_PATH selects another build of the library (the host-sanitized copy of the CPU tests)
LIB_PATH = os.environ.get("LIBTTT_PATH") or os.path.join(PKG, "libttt.so")

FW = {"swiglu": 0, "gelu": 1, "linear": 2}
LOSS = {"dot": 0, "mse": 1}
ACT = {"f32": 0, "bf16": 1}
ORDER = {"apply_then_update": 0, "update_then_apply": 1}

STATUS = {0: "TTT_OK", 1: "TTT_E_NULL", 2: "TTT_E_SHAPE", 3: "TTT_E_DTYPE", 4: "TTT_E_CONFIG",
          5: "TTT_E_UNSUPPORTED", 6: "TTT_E_ALLOC", 7: "TTT_E_HIP", 8: "TTT_E_NONFINITE",
          9: "TTT_E_ALIGN"}

# bf16 planes per operand class (apply, grad, ns) and the mask of Newton-Schulz iterations
# run on one plane (ns_one_plane) for the named workloads; chosen as the cheapest setting
# whose end-to-end error stays well inside the parity bound.
PRECISION = {
    "tiny": (3, 3, 3, 0),
    "lm": (1, 2, 2, 0b00011),
    "long": (1, 3, 3, 0),
    "long_alt": (1, 3, 3, 0),
    "imageset": (1, 1, 2, 0),
    "smallchunk": (1, 1, 1, 0),
}


class TTTError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class ttt_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "heads", "dim", "hidden", "chunk", "fw", "loss", "act", "order", "ns_steps",
        "row_renorm", "apply_planes", "grad_planes", "ns_planes", "ns_one_plane", "path")
    ] + [("lr", ctypes.c_float * 3), ("weight_decay", ctypes.c_float), ("replay", ctypes.c_int32),
         ("momentum", ctypes.c_float)]


class ttt_block_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "dim", "window", "window_mode", "ffn_hidden", "reserved")
    ] + [("max_seq_len", ctypes.c_int64), ("ttt", ttt_config)]


BLOCK_WEIGHTS = ("attn_qkv", "attn_out", "ttt_qkv", "ttt_eta", "ttt_out", "ffn_up", "ffn_down")


class ttt_block_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BLOCK_WEIGHTS]


WINDOW = {"sliding": 0, "block": 1}
LINEAR_EPI = {"plain": 0, "residual": 1, "gelu": 2}
ATTN_HEAD_DIM = 128

_lib = None


def lib() -> ctypes.CDLL:
    """Load libttt.so (built in-tree by build.py). Raises if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run weight_sequence_layers_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        cfgp, vp, i64 = ctypes.POINTER(ttt_config), ctypes.c_void_p, ctypes.c_int64
        i32 = ctypes.c_int32
        sig = {
            "ttt_validate_config": [cfgp],
            "ttt_state_numel": [cfgp, ctypes.POINTER(i64)],
            "ttt_init_state": [cfgp, vp, vp, ctypes.POINTER(vp)],
            "ttt_chunk_forward": [vp, vp, vp, vp, vp, vp, vp],
            "ttt_sequence_forward": [vp, vp, vp, vp, vp, vp, i64, vp],
            "ttt_sequence_forward_masked": [vp, vp, vp, vp, vp, vp, i64, vp, vp],
            "ttt_apply_backward": [vp, vp, vp, vp, vp, vp],
            "ttt_chunk_backward": [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
            "ttt_get_state": [vp, vp, vp],
            "ttt_set_state": [vp, vp, vp],
            "ttt_state_health": [vp],
            "ttt_destroy_state": [vp],
            "ttt_sequence_forward_noalloc": [cfgp, vp, vp, vp, vp, vp, vp, i64, vp],
            "ttt_profile_begin": [vp, ctypes.c_int32, ctypes.c_int32],
            "ttt_profile_end": [vp, ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_double)],
            "ttt_window_attention": [vp, vp, vp, i64, vp, i64, i32, i32, i64, i32, i32, vp],
            "ttt_linear": [vp, vp, vp, vp, i64, i32, i32, i32, vp],
            "ttt_block_init": [ctypes.POINTER(ttt_block_config),
                               ctypes.POINTER(ttt_block_weights), vp, vp, ctypes.POINTER(vp)],
            "ttt_block_forward": [vp, vp, vp, i64, vp],
            "ttt_block_destroy": [vp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.ttt_block_ttt_state.argtypes = [vp]
        L.ttt_block_ttt_state.restype = vp
        L.ttt_status_str.argtypes = [ctypes.c_int]
        L.ttt_status_str.restype = ctypes.c_char_p
        L.ttt_last_error.argtypes = []
        L.ttt_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(st: int):
    if st != 0:
        raise TTTError(st, lib().ttt_last_error().decode())


PATH = {"auto": 0, "staged": 1, "resident": 2}


def make_config(cfg=None, *, planes=None, **kw) -> ttt_config:
    """ttt_config from an object with the workload fields (batch, heads, dim, hidden, chunk,
    fw, loss, act, order, ns_steps, renorm and optionally lr, weight_decay), overridden by
    keyword arguments. `planes` is (apply, grad, ns, ns_one_plane); by default the preset of
    the workload's name, else 0s. `path` is "auto", "staged" or "resident". `lr` is a
    sequence of up to 3 step sizes in the state's matrix order (0 or missing: 1). `replay`
    records each call's launches in a HIP graph and replays it for repeated pointers."""
    f = {}
    if cfg is not None:
        for k in ("batch", "heads", "dim", "hidden", "chunk", "fw", "loss", "act", "order",
                  "ns_steps", "renorm"):
            f[k] = getattr(cfg, k)
        for k in ("lr", "weight_decay", "momentum"):
            if hasattr(cfg, k):
                f[k] = getattr(cfg, k)
        if planes is None:
            planes = PRECISION.get(getattr(cfg, "name", ""), None)
    f.update(kw)
    planes = planes or (0, 0, 0, 0)
    c = ttt_config()
    c.batch, c.heads, c.dim, c.hidden, c.chunk = (int(f["batch"]), int(f["heads"]), int(f["dim"]),
                                                  int(f["hidden"]), int(f["chunk"]))
    c.fw = FW[f["fw"]] if isinstance(f["fw"], str) else int(f["fw"])
    c.loss = LOSS[f["loss"]] if isinstance(f["loss"], str) else int(f["loss"])
    c.act = ACT[f["act"]] if isinstance(f["act"], str) else int(f["act"])
    c.order = ORDER[f["order"]] if isinstance(f["order"], str) else int(f["order"])
    c.ns_steps = int(f.get("ns_steps", 0))
    c.row_renorm = int(bool(f.get("renorm", False)))
    c.apply_planes, c.grad_planes, c.ns_planes, c.ns_one_plane = (int(p) for p in planes)
    path = f.get("path", "auto")
    c.path = PATH[path] if isinstance(path, str) else int(path)
    lr = list(f.get("lr", ()) or ())
    if len(lr) > 3:
        raise ValueError("at most 3 step sizes")
    for i, x in enumerate(lr):
        c.lr[i] = float(x)
    c.weight_decay = float(f.get("weight_decay", 0.0))
    c.replay = int(bool(f.get("replay", False)))
    c.momentum = float(f.get("momentum", 0.0))
    return c


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return int(getattr(stream, "cuda_stream", stream)) or None


def ttt_validate_config(cfg: ttt_config) -> None:
    _check(lib().ttt_validate_config(ctypes.byref(cfg)))


def ttt_state_numel(cfg: ttt_config) -> int:
    n = ctypes.c_int64()
    _check(lib().ttt_state_numel(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


class State:
    """Owns a ttt_state handle (freed by destroy() or garbage collection), or, with
    owner set, refers to one that object owns (destroy() then only drops the reference)."""

    def __init__(self, handle: int, cfg: ttt_config, owner=None):
        self.handle = ctypes.c_void_p(handle)
        self.cfg = cfg
        self.owner = owner

    def destroy(self):
        if self.handle:
            h, self.handle = self.handle, None
            if self.owner is None:
                _check(lib().ttt_destroy_state(h))

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def ttt_init_state(cfg: ttt_config, w0, stream=None) -> State:
    """w0: contiguous fp32 device tensor with the per-head initial matrices, matrix by
    matrix (see include/libttt.h)."""
    h = ctypes.c_void_p()
    _check(lib().ttt_init_state(ctypes.byref(cfg), _ptr(w0), _stream(stream), ctypes.byref(h)))
    return State(h.value, cfg)


def ttt_chunk_forward(st: State, q, k, v, eta, out, stream=None) -> None:
    _check(lib().ttt_chunk_forward(st.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(out),
                                   _stream(stream)))


def ttt_apply_backward(st: State, q, dout, dq, dw, stream=None) -> None:
    """Backward of one chunk's apply step with the state as it stands: dq [B,H,chunk,d] and
    dw (state-shaped fp32) of sum <dout, f_W(q)> (see include/libttt.h)."""
    _check(lib().ttt_apply_backward(st.handle, _ptr(q), _ptr(dout), _ptr(dq), _ptr(dw),
                                    _stream(stream)))


def ttt_chunk_backward(st: State, q, k, v, eta, dout, dw, dq, dk, dv, deta, stream=None) -> None:
    """Backward through one chunk with the state as it stands (the state before the chunk):
    dw holds the cotangent of the state after the chunk and receives that of the state
    before it; dq, dk, dv, deta receive the input gradients (see include/libttt.h)."""
    _check(lib().ttt_chunk_backward(st.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(dout),
                                    _ptr(dw), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(deta),
                                    _stream(stream)))


def ttt_sequence_forward(st: State, q, k, v, eta, out, seq_len: int, stream=None) -> None:
    _check(lib().ttt_sequence_forward(st.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
                                      _ptr(out), int(seq_len), _stream(stream)))


# workspace bytes the allocation-free call holds per GPU (TTT_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


def ttt_sequence_forward_noalloc(cfg: ttt_config, state, q, k, v, eta, out, seq_len: int,
                                 stream=None) -> None:
    """ttt_sequence_forward with no state object and no allocation: `state` (fp32 device
    tensor, the ttt_get_state layout) holds the initial weights and receives the final ones
    (see include/libttt.h)."""
    _check(lib().ttt_sequence_forward_noalloc(ctypes.byref(cfg), _ptr(state), _ptr(q), _ptr(k),
                                              _ptr(v), _ptr(eta), _ptr(out), int(seq_len),
                                              _stream(stream)))


def ttt_sequence_forward_masked(st: State, q, k, v, eta, out, seq_len: int, update,
                                stream=None) -> None:
    """ttt_sequence_forward in which chunk c updates the state only if update[c] is true
    (a sequence of seq_len/chunk flags, or None for all; see include/libttt.h)."""
    n = int(seq_len) // st.cfg.chunk
    arr = None
    if update is not None:
        flags = [1 if u else 0 for u in update]
        if len(flags) != n:
            raise ValueError(f"{len(flags)} update flags for {n} chunks")
        arr = (ctypes.c_uint8 * max(n, 1))(*flags)
    _check(lib().ttt_sequence_forward_masked(st.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
                                             _ptr(out), int(seq_len),
                                             ctypes.cast(arr, ctypes.c_void_p) if arr else None,
                                             _stream(stream)))


def ttt_get_state(st: State, dst, stream=None) -> None:
    _check(lib().ttt_get_state(st.handle, _ptr(dst), _stream(stream)))


def ttt_set_state(st: State, src, stream=None) -> None:
    _check(lib().ttt_set_state(st.handle, _ptr(src), _stream(stream)))


def ttt_state_health(st: State) -> None:
    _check(lib().ttt_state_health(st.handle))


def ttt_destroy_state(st: State) -> None:
    st.destroy()


STAGES = {"front_q": 0, "front_k": 1, "out": 2, "contract": 3, "ns_gram": 4, "ns_poly": 5,
          "ns_update": 6, "renorm": 7, "split": 8, "mse": 9, "resident": 10, "dq": 11,
          "tfront": 12, "ns_bwd": 13, "ns_small": 14}


def ttt_profile_begin(st: State, stage, max_launches: int = 4096) -> None:
    """Bracket every launch of one stage kernel with HIP events (see include/libttt.h)."""
    sid = STAGES[stage] if isinstance(stage, str) else int(stage)
    _check(lib().ttt_profile_begin(st.handle, sid, int(max_launches)))


def ttt_profile_end(st: State):
    """Returns (timed launches, total milliseconds)."""
    n = ctypes.c_int64()
    ms = ctypes.c_double()
    _check(lib().ttt_profile_end(st.handle, ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def matrix_shapes(cfg: ttt_config):
    d, dh = cfg.dim, cfg.hidden
    return {0: [(dh, d), (dh, d), (d, dh)], 1: [(dh, d), (d, dh)], 2: [(d, d)]}[cfg.fw]


def split_state(cfg: ttt_config, flat):
    """Views of a flat state buffer as per-matrix [batch, heads, rows, cols] tensors: the
    fast weights, then (with momentum) their buffers."""
    out, o = [], 0
    shapes = matrix_shapes(cfg)
    for r, c in shapes + (shapes if cfg.momentum > 0 else []):
        n = cfg.batch * cfg.heads * r * c
        out.append(flat[o:o + n].view(cfg.batch, cfg.heads, r, c))
        o += n
    return out


# ---------------------------------------------------------------- the LaCT block (ttt_block.h)
def ttt_window_attention(q, k, v, ld: int, out, ld_out: int, batch: int, heads: int,
                         seq_len: int, window: int, mode="sliding", stream=None) -> None:
    """Window attention over heads of 128: q, k, v, out bf16 device tensors whose element
    (b, t, h, e) sits at (b seq_len + t) ld + 128 h + e (ld_out for out); mode "sliding" or
    "block" (see include/ttt_block.h)."""
    m = WINDOW[mode] if isinstance(mode, str) else int(mode)
    _check(lib().ttt_window_attention(_ptr(q), _ptr(k), _ptr(v), int(ld), _ptr(out),
                                      int(ld_out), int(batch), int(heads), int(seq_len),
                                      int(window), m, _stream(stream)))


def ttt_linear(x, w, resid, y, rows: int, in_features: int, out_features: int,
               epilogue="plain", stream=None) -> None:
    """y = epilogue(x w^T) in bf16 with fp32 accumulation; epilogue "plain", "residual"
    (adds resid) or "gelu" (see include/ttt_block.h)."""
    e = LINEAR_EPI[epilogue] if isinstance(epilogue, str) else int(epilogue)
    _check(lib().ttt_linear(_ptr(x), _ptr(w), _ptr(resid), _ptr(y), int(rows), int(in_features),
                            int(out_features), e, _stream(stream)))


def make_block_config(ttt: ttt_config, *, dim: int, window: int, mode="sliding",
                      ffn_hidden: int = 0, max_seq_len: int) -> ttt_block_config:
    c = ttt_block_config()
    c.batch = ttt.batch
    c.dim = int(dim)
    c.window = int(window)
    c.window_mode = WINDOW[mode] if isinstance(mode, str) else int(mode)
    c.ffn_hidden = int(ffn_hidden)
    c.reserved = 0
    c.max_seq_len = int(max_seq_len)
    c.ttt = ttt
    return c


class Block:
    """Owns a ttt_block handle and keeps the weight tensors it references alive."""

    def __init__(self, handle: int, cfg: ttt_block_config, weights):
        self.handle = ctypes.c_void_p(handle)
        self.cfg = cfg
        self.weights = weights

    def destroy(self):
        if self.handle:
            h, self.handle = self.handle, None
            _check(lib().ttt_block_destroy(h))

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def ttt_block_init(cfg: ttt_block_config, weights, w0, stream=None) -> Block:
    """weights: mapping from the names in BLOCK_WEIGHTS to contiguous bf16 device tensors;
    w0: the TTT sub-layer's initial matrices (the layout ttt_init_state takes)."""
    w = ttt_block_weights()
    for n in BLOCK_WEIGHTS:
        setattr(w, n, _ptr(weights[n]))
    h = ctypes.c_void_p()
    _check(lib().ttt_block_init(ctypes.byref(cfg), ctypes.byref(w), _ptr(w0), _stream(stream),
                                ctypes.byref(h)))
    return Block(h.value, cfg, dict(weights))


def ttt_block_forward(blk: Block, x, y, seq_len: int, stream=None) -> None:
    _check(lib().ttt_block_forward(blk.handle, _ptr(x), _ptr(y), int(seq_len), _stream(stream)))


def ttt_block_ttt_state(blk: Block) -> State:
    """The block's TTT state, for ttt_get_state and the other state calls."""
    return State(lib().ttt_block_ttt_state(blk.handle), blk.cfg.ttt, owner=blk)


def ttt_block_destroy(blk: Block) -> None:
    blk.destroy()
