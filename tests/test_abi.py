"""The C-ABI library: it loads, exports every function the header declares, and rejects bad
arguments on the host before touching a GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import weight_sequence_layers_amd as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libttt.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


def _declared(path=HEADER):
    src = open(path).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ttt_[a-z_0-9]+)\s*\(", src)))


@pytest.mark.parametrize("header", HEADERS, ids=os.path.basename)
def test_library_exports_every_declared_function(header):
    L = W.lib()
    names = _declared(header)
    assert names
    for n in names:
        assert hasattr(L, n), n


def _cfg(**kw):
    base = dict(batch=2, heads=2, dim=64, hidden=128, chunk=64, fw="swiglu", loss="dot",
                act="bf16", order="apply_then_update", ns_steps=5, renorm=True)
    base.update(kw)
    return W.make_config(None, **base)


def _status(cfg):
    return W.lib().ttt_validate_config(ctypes.byref(cfg))


def test_valid_configs_pass():
    for kw in [{}, dict(fw="gelu", loss="mse", ns_steps=0, renorm=False), dict(fw="linear"),
               dict(act="f32"), dict(order="update_then_apply", chunk=1 << 30),
               dict(dim=16, hidden=16), dict(dim=1024, hidden=4096)]:
        assert _status(_cfg(**kw)) == 0, kw
    W.ttt_validate_config(_cfg())


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), 2), (dict(heads=-1), 2), (dict(batch=300, heads=300), 2),
    (dict(dim=8), 2), (dict(dim=72), 2), (dict(dim=2048, hidden=4096), 2),
    (dict(hidden=100), 2), (dict(hidden=8192), 2), (dict(chunk=0), 2),
    (dict(fw=7), 4), (dict(loss=2), 4), (dict(act=5), 3), (dict(order=-1), 4),
    (dict(ns_steps=9), 4), (dict(dim=256, hidden=128), 5),
])
def test_invalid_configs_rejected(kw, code):
    assert _status(_cfg(**kw)) == code
    with pytest.raises(W.TTTError) as e:
        W.ttt_validate_config(_cfg(**kw))
    assert e.value.status == code and len(str(e.value)) > 12


@pytest.mark.parametrize("kw,ok", [
    (dict(lr=(0.5, 2.0, 0.0)), True), (dict(lr=(0.0,)), True), (dict(weight_decay=0.0), True),
    (dict(weight_decay=0.999), True), (dict(lr=(1.0, -0.1)), False),
    (dict(lr=(float("nan"),)), False), (dict(lr=(1.0, 1.0, float("inf"))), False),
    (dict(weight_decay=1.0), False), (dict(weight_decay=-1e-3), False),
    (dict(weight_decay=float("nan")), False),
])
def test_step_size_and_decay_checked(kw, ok):
    assert _status(_cfg(**kw)) == (0 if ok else 4), kw


def test_step_size_fields_reach_the_struct():
    c = _cfg(lr=(0.25, 0.5), weight_decay=0.125)
    assert list(c.lr) == [0.25, 0.5, 0.0] and c.weight_decay == 0.125
    assert ctypes.sizeof(W.ttt_config) == 16 * 4 + 4 * 4 + 4 + 4


def test_momentum_checked_and_counted_in_the_state():
    for beta, code in ((0.0, 0), (0.5, 0), (0.999, 0), (1.0, 4), (-0.1, 4),
                       (float("nan"), 4)):
        assert _status(_cfg(momentum=beta)) == code, beta
    assert W.ttt_state_numel(_cfg(momentum=0.9)) == 2 * W.ttt_state_numel(_cfg())
    small = dict(fw="gelu", loss="mse", ns_steps=0, renorm=False, dim=64, hidden=256, chunk=64)
    assert _status(W.make_config(None, planes=(1, 1, 1, 0), path="resident", momentum=0.5,
                                 **_base(**small))) == 5
    c = W.make_config(None, planes=(1, 1, 1, 0), momentum=0.5, **_base(**small))
    assert _status(c) == 0


def test_replay_flag_checked():
    c = _cfg()
    for val, code in ((0, 0), (1, 0), (2, 4), (-1, 4)):
        c.replay = val
        assert _status(c) == code, val
    assert W.make_config(None, replay=True, **_base()).replay == 1


def test_plane_counts_checked():
    c = _cfg()
    c.grad_planes = 4
    assert _status(c) == 4
    c.grad_planes = -1
    assert _status(c) == 4
    c.grad_planes = 3
    assert _status(c) == 0


def test_one_plane_mask_checked():
    c = _cfg()
    for mask, code in ((0, 0), (3, 0), (255, 0), (256, 4), (-1, 4)):
        c.ns_one_plane = mask
        assert _status(c) == code, mask


def test_null_config_and_pointers():
    L = W.lib()
    assert L.ttt_validate_config(None) == 1
    h = ctypes.c_void_p()
    assert L.ttt_init_state(ctypes.byref(_cfg()), None, None, ctypes.byref(h)) == 1
    assert h.value is None
    assert L.ttt_init_state(ctypes.byref(_cfg()), 0x1008, None, ctypes.byref(h)) == 9
    assert L.ttt_init_state(ctypes.byref(_cfg()), 0x1000, None, None) == 1
    assert L.ttt_chunk_forward(None, 16, 16, 16, 16, 16, None) == 1
    assert L.ttt_sequence_forward(None, 16, 16, 16, 16, 16, 64, None) == 1
    assert L.ttt_sequence_forward_masked(None, 16, 16, 16, 16, 16, 64, None, None) == 1
    assert L.ttt_get_state(None, 16, None) == 1
    assert L.ttt_set_state(None, 16, None) == 1
    assert L.ttt_state_health(None) == 1
    assert L.ttt_destroy_state(None) == 0
    assert b"NULL" in L.ttt_last_error() or len(L.ttt_last_error()) > 0


def test_state_numel():
    assert W.ttt_state_numel(_cfg()) == 2 * 2 * 3 * 64 * 128
    assert W.ttt_state_numel(_cfg(fw="gelu")) == 2 * 2 * 2 * 64 * 128
    assert W.ttt_state_numel(_cfg(fw="linear")) == 2 * 2 * 64 * 64


def test_status_strings():
    L = W.lib()
    for code in range(10):
        s = L.ttt_status_str(code)
        assert s and s != b"unknown status"
    assert L.ttt_status_str(99) == b"unknown status"


def test_path_selection_checked():
    small = dict(fw="gelu", loss="mse", ns_steps=0, renorm=False, dim=64, hidden=256, chunk=64)
    one = (1, 1, 1, 0)
    # the resident loop serves the small-chunk GELU layer with one bf16 plane
    for kw in [small, dict(small, chunk=1), dict(small, chunk=48), dict(small, loss="dot")]:
        assert _status(W.make_config(None, planes=one, path="resident", **_base(**kw))) == 0, kw
    # and nothing else
    for kw in [dict(small, chunk=65), dict(small, dim=128), dict(small, hidden=512),
               dict(small, ns_steps=5, renorm=True), dict(small, renorm=True),
               dict(small, act="f32"), dict(small, order="update_then_apply"),
               dict(small, fw="swiglu")]:
        assert _status(W.make_config(None, planes=one, path="resident", **_base(**kw))) == 5, kw
    # two gradient planes (the bf16 default) keep the staged kernels
    assert _status(W.make_config(None, planes=(1, 2, 2, 0), path="resident",
                                 **_base(**small))) == 5
    for path in ("auto", "staged"):
        assert _status(W.make_config(None, planes=(1, 2, 2, 0), path=path,
                                     **_base(**small))) == 0
    c = _cfg()
    c.path = 3
    assert _status(c) == 4


def _base(**kw):
    base = dict(batch=2, heads=2, dim=64, hidden=128, chunk=64, fw="swiglu", loss="dot",
                act="bf16", order="apply_then_update", ns_steps=5, renorm=True)
    base.update(kw)
    return base


def test_noalloc_call_rejects_on_the_host():
    """The allocation-free call checks its arguments and its workspace limit before any HIP
    call, so these run without a GPU: the LaCT language-model layer (8 problems of dim 512,
    hidden 1024) needs more workspace than the call holds."""
    L = W.lib()
    lm = _cfg(batch=4, heads=2, dim=512, hidden=1024, chunk=2048)
    p = 0x10000
    assert L.ttt_sequence_forward_noalloc(ctypes.byref(lm), p, p, p, p, p, p, 4096, None) == 2
    msg = L.ttt_last_error().decode()
    assert "workspace" in msg and str(W.NOALLOC_SCRATCH_BYTES) in msg
    small = _cfg()
    assert L.ttt_sequence_forward_noalloc(None, p, p, p, p, p, p, 64, None) == 1
    assert L.ttt_sequence_forward_noalloc(ctypes.byref(small), None, p, p, p, p, p, 64, None) == 1
    assert L.ttt_sequence_forward_noalloc(ctypes.byref(small), p + 8, p, p, p, p, p, 64, None) == 9
    assert L.ttt_sequence_forward_noalloc(ctypes.byref(small), p, p, p, p, p, p, 65, None) == 2
    assert L.ttt_sequence_forward_noalloc(ctypes.byref(small), p, None, p, p, p, p, 64, None) == 1
    assert L.ttt_sequence_forward_noalloc(ctypes.byref(_cfg(dim=72)), p, p, p, p, p, p, 64,
                                          None) == 2


def test_noalloc_limit_matches_the_header():
    m = re.search(r"#define\s+TTT_NOALLOC_SCRATCH_BYTES\s+(\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == W.NOALLOC_SCRATCH_BYTES


def test_block_struct_layout():
    """ttt_block_config: six int32 fields, the int64 max_seq_len, then the layer's config."""
    assert ctypes.sizeof(W.ttt_block_config) == 6 * 4 + 8 + ctypes.sizeof(W.ttt_config)
    assert W.ttt_block_config.ttt.offset == 32
    assert ctypes.sizeof(W.ttt_block_weights) == 7 * ctypes.sizeof(ctypes.c_void_p)


def test_block_calls_reject_on_the_host():
    """Every block call checks its arguments before any HIP call."""
    L = W.lib()
    p = 0x10000
    # window attention: heads of 128 need ld >= heads * 128; unknown mode; window 0
    assert L.ttt_window_attention(p, p, p, 128, p, 128, 1, 2, 64, 8, 0, None) == 2
    assert L.ttt_window_attention(p, p, p, 384, p, 128, 1, 1, 64, 8, 2, None) == 4
    assert L.ttt_window_attention(p, p, p, 384, p, 128, 1, 1, 64, 0, 0, None) == 2
    assert L.ttt_window_attention(p, p, p, 388, p, 128, 1, 1, 64, 8, 0, None) == 2
    assert L.ttt_window_attention(None, p, p, 384, p, 128, 1, 1, 64, 8, 0, None) == 1
    assert L.ttt_window_attention(p + 2, p, p, 384, p, 128, 1, 1, 64, 8, 0, None) == 9
    assert L.ttt_window_attention(None, None, None, 384, None, 128, 1, 1, 0, 8, 0, None) == 0
    # the output inside the inputs' rows (in place over q, or over v's third of the rows)
    assert L.ttt_window_attention(p, p + 256, p + 512, 384, p, 128, 1, 1, 64, 8, 0, None) == 4
    assert L.ttt_window_attention(p, p + 256, p + 512, 384, p + 512, 384, 1, 1, 64, 8, 0,
                                  None) == 4
    # projections: feature counts multiples of 8; epilogue; residual pointer; overlap
    assert L.ttt_linear(p, p, None, p, 4, 12, 8, 0, None) == 2
    assert L.ttt_linear(p, p, None, p, 4, 8, 12, 0, None) == 2
    assert L.ttt_linear(p, p, None, p, 4, 8, 8, 3, None) == 4
    assert L.ttt_linear(p, p, None, p + 4096, 4, 8, 8, 1, None) == 1
    assert L.ttt_linear(p, p + 4096, None, p, 4, 8, 8, 0, None) == 4
    assert L.ttt_linear(None, None, None, None, 0, 8, 8, 0, None) == 0
    # block configs
    t = _cfg(batch=2, heads=2, dim=128, hidden=256, chunk=64)
    w = W.ttt_block_weights(*([p] * 7))
    h = ctypes.c_void_p()

    def init(**kw):
        c = W.make_block_config(t, **{**dict(dim=256, window=64, max_seq_len=256), **kw})
        return L.ttt_block_init(ctypes.byref(c), ctypes.byref(w), p, None, ctypes.byref(h))
    assert init(dim=192) == 2                  # not a multiple of 128
    assert init(dim=384) == 2                  # ttt.heads * ttt.dim differs
    assert init(window=0) == 2
    assert init(mode=5) == 4
    assert init(ffn_hidden=12) == 2
    c = W.make_block_config(t, dim=256, window=64, max_seq_len=256)
    c.reserved = 1
    assert L.ttt_block_init(ctypes.byref(c), ctypes.byref(w), p, None, ctypes.byref(h)) == 4
    c32 = W.make_block_config(_cfg(batch=2, heads=2, dim=128, hidden=256, chunk=64, act="f32"),
                              dim=256, window=64, max_seq_len=256)
    assert L.ttt_block_init(ctypes.byref(c32), ctypes.byref(w), p, None, ctypes.byref(h)) == 3
    wb = W.ttt_block_weights(*([p] * 6 + [None]))
    c = W.make_block_config(t, dim=256, window=64, max_seq_len=256)
    assert L.ttt_block_init(ctypes.byref(c), ctypes.byref(wb), p, None, ctypes.byref(h)) == 1
    assert h.value is None
    assert L.ttt_block_forward(None, p, p, 64, None) == 1
    assert L.ttt_block_destroy(None) == 0
    assert L.ttt_block_ttt_state(None) is None
