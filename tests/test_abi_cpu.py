"""Host-side checks of the C-ABI library (no GPU work is launched).

The library must load, export every entry point include/albert.h declares,
and answer the host-only queries (configuration, tensor names and shapes,
status strings, argument rejection) without touching a device.
"""
import ctypes
import os
import re

import numpy as np

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "albert.h")


@pytest.fixture(scope="module")
def L():
    import torch  # noqa: F401  (shares its HIP runtime with the library)
    import albert_transformer_amd as A
    return A.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(albert_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    import albert_transformer_amd as A
    assert declared_functions() == sorted(A.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_default_config_and_tensor_table(L):
    import albert_transformer_amd as A
    c = A.default_config()
    k = synth.KOKORO
    for f in ("vocab", "max_pos", "n_types", "emb", "hidden", "heads", "head_dim",
              "ffn", "n_iter", "n_groups", "out_dim"):
        assert getattr(c, f) == getattr(k, f), f
    assert abs(c.ln_eps - 1e-12) < 1e-18
    assert L.albert_n_tensors(ctypes.byref(c)) == len(synth.TENSOR_NAMES) == 25
    shapes = k.shapes()
    for i, name in enumerate(synth.TENSOR_NAMES):
        assert L.albert_tensor_name(ctypes.byref(c), i).decode() == name
        r, cc = ctypes.c_int64(), ctypes.c_int64()
        assert L.albert_tensor_shape(ctypes.byref(c), i, ctypes.byref(r), ctypes.byref(cc)) == 0
        shp = shapes[name]
        assert (r.value, cc.value) == (shp[0], shp[1] if len(shp) == 2 else 1)
    assert L.albert_tensor_name(ctypes.byref(c), 25) is None
    assert L.albert_tensor_name(ctypes.byref(c), -1) is None


@pytest.mark.parametrize("G", [2, 3, 12])
def test_grouped_tensor_table(L, G):
    """With G weight sets the layer tensors repeat per set, in the order
    synth.tensor_names draws them."""
    import albert_transformer_amd as A
    c = A.default_config(n_groups=G)
    cfg = synth.Config(n_groups=G)
    names = synth.tensor_names(cfg)
    assert L.albert_n_tensors(ctypes.byref(c)) == len(names) == 9 + 16 * G
    shapes = cfg.shapes()
    for i, name in enumerate(names):
        assert L.albert_tensor_name(ctypes.byref(c), i).decode() == synth.base_name(name)
        r, cc = ctypes.c_int64(), ctypes.c_int64()
        assert L.albert_tensor_shape(ctypes.byref(c), i, ctypes.byref(r), ctypes.byref(cc)) == 0
        shp = shapes[synth.base_name(name)]
        assert (r.value, cc.value) == (shp[0], shp[1] if len(shp) == 2 else 1)
    assert L.albert_tensor_name(ctypes.byref(c), len(names)) is None


def test_config_rejections(L):
    import albert_transformer_amd as A
    r, cc = ctypes.c_int64(), ctypes.c_int64()
    for bad in (dict(hidden=1024), dict(heads=8), dict(ffn=1000), dict(out_dim=100),
                dict(max_pos=513), dict(n_iter=-1), dict(emb=64), dict(n_groups=0),
                dict(n_groups=13), dict(n_iter=4, n_groups=5)):
        c = A.default_config(**bad)
        assert L.albert_tensor_shape(ctypes.byref(c), 0, ctypes.byref(r), ctypes.byref(cc)) == A.E_ARG
        assert L.albert_n_tensors(ctypes.byref(c)) == -1
    # n_iter = 0 keeps one weight set
    assert L.albert_n_tensors(ctypes.byref(A.default_config(n_iter=0))) == 25
    h = ctypes.c_void_p()
    ptrs = (ctypes.c_void_p * 25)()
    c = A.default_config(hidden=1024)
    assert L.albert_load_weights(ctypes.byref(h), ctypes.byref(c), ptrs, 1, None) == A.E_ARG
    assert h.value is None


def test_null_context_is_rejected_without_device_work(L):
    import albert_transformer_amd as A
    assert L.albert_workspace_bytes(None, 4, 512) == 0
    assert L.albert_encode(None, None, None, 1, 8, None, None, 0, None, 0) == A.E_ARG
    assert L.albert_encode_varlen(None, None, None, 1, 8, 8, None, None, 0, None, 0) == A.E_ARG
    assert L.albert_read_status(None, None) == A.E_ARG
    off, nb, st = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int64()
    assert L.albert_tap(None, 1, 1, 0, ctypes.byref(off), ctypes.byref(nb), ctypes.byref(st)) == A.E_ARG
    L.albert_free(None)


def test_status_strings(L):
    import albert_transformer_amd as A
    for code in A.STATUS_NAMES:
        assert A.status_str(code)
    assert A.status_str(99) == "unknown status"


def test_text_encoder_tensor_table(L):
    """The text path's tensor names and shapes follow synth.TextConfig."""
    import albert_transformer_amd as A
    c = A.text_default_config()
    k = synth.TEXT
    for f in ("vocab", "channels", "kernel", "n_conv", "hidden"):
        assert getattr(c, f) == getattr(k, f), f
    names = k.tensor_names()
    assert L.albert_text_n_tensors(ctypes.byref(c)) == len(names) == 24
    shapes = k.shapes()
    for i, name in enumerate(names):
        assert L.albert_text_tensor_name(ctypes.byref(c), i).decode() == name
        r, cc = ctypes.c_int64(), ctypes.c_int64()
        assert L.albert_text_tensor_shape(ctypes.byref(c), i, ctypes.byref(r), ctypes.byref(cc)) == 0
        assert r.value * cc.value == int(np.prod(shapes[name])) and r.value == shapes[name][0]
    assert L.albert_text_tensor_name(ctypes.byref(c), len(names)) is None
    for bad in (dict(channels=256), dict(kernel=4), dict(kernel=9), dict(n_conv=0),
                dict(n_conv=9), dict(hidden=128), dict(ln_eps=0.0)):
        assert L.albert_text_n_tensors(ctypes.byref(A.text_default_config(**bad))) == -1
    assert L.albert_text_workspace_bytes(None, 1, 1) == 0
    assert L.albert_text_encode(None, None, None, 1, 8, None, None, 0, None, 0) == A.E_ARG
    L.albert_text_free(None)


def test_binding_refuses_tensors_the_library_would_misread():
    """The library sees bare pointers: the binding checks element type,
    device and contiguity first (an int64 ID tensor would otherwise be read
    as pairs of in-range int32 values and return OK)."""
    import torch
    from albert_transformer_amd._lib import _need
    with pytest.raises(ValueError, match="int32"):
        _need(torch.zeros(4, dtype=torch.int64), "ids", torch.int32)
    with pytest.raises(ValueError, match="device"):
        _need(torch.zeros(4, dtype=torch.int32), "ids", torch.int32)
    with pytest.raises(TypeError):
        _need(np.zeros(4, np.int32), "ids", torch.int32)


def test_scratch_size_matches_the_header():
    import albert_transformer_amd as A
    text = open(HEADER).read()
    m = re.search(r"#define ALBERT_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == A.SCRATCH_BYTES
    assert re.search(r"ALBERT_E_SCRATCH = (\d+)", text).group(1) == str(A.E_SCRATCH)
