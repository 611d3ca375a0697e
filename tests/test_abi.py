"""The C-ABI library: it loads, exports every function the header declares, and rejects bad
arguments on the host before touching a GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import weight_sequence_layers_amd as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libttt.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ttt_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    L = W.lib()
    names = _declared()
    assert "ttt_init_state" in names and "ttt_sequence_forward" in names
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
    assert ctypes.sizeof(W.ttt_config) == 16 * 4 + 4 * 4


def test_plane_counts_checked():
    c = _cfg()
    c.grad_planes = 4
    assert _status(c) == 4
    c.grad_planes = -1
    assert _status(c) == 4
    c.grad_planes = 3
    assert _status(c) == 0


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
    one = (1, 1, 1, 1)
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
    assert _status(W.make_config(None, planes=(1, 2, 2, 2), path="resident",
                                 **_base(**small))) == 5
    for path in ("auto", "staged"):
        assert _status(W.make_config(None, planes=(1, 2, 2, 2), path=path,
                                     **_base(**small))) == 0
    c = _cfg()
    c.path = 3
    assert _status(c) == 4


def _base(**kw):
    base = dict(batch=2, heads=2, dim=64, hidden=128, chunk=64, fw="swiglu", loss="dot",
                act="bf16", order="apply_then_update", ns_steps=5, renorm=True)
    base.update(kw)
    return base
