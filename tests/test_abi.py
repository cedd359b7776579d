"""The C-ABI library: it loads, exports every function include/flint_moe.h
declares, and rejects invalid arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import int4_expert_ffn_amd as F

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "flint_moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flint_moe_\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(F.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = F.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_constants_match_header():
    text = open(HEADER).read()
    for name in ("FLINT_HIDDEN", "FLINT_EXPERTS", "FLINT_EXPERT_SIZE", "FLINT_SHARED_SIZE", "FLINT_TOP_K",
                 "FLINT_GROUP", "FLINT_MAX_LAYERS", "FLINT_MAX_TOKENS", "FLINT_OK", "FLINT_ERR_INVALID_ARG",
                 "FLINT_ERR_OUT_OF_MEMORY", "FLINT_ERR_HIP", "FLINT_ERR_UNSUPPORTED", "FLINT_ERR_DEVICE"):
        m = re.search(r"#define\s+%s\s+(-?\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(F, name), name


def test_create_rejects_bad_arguments_before_any_hip_call():
    lib = F.lib()
    h = ctypes.c_void_p(1234)
    assert lib.flint_moe_create(None, 1, ctypes.byref(h)) == F.FLINT_ERR_INVALID_ARG
    assert h.value is None
    layer = (F.flint_moe_layer * 1)()
    assert lib.flint_moe_create(layer, 0, ctypes.byref(h)) == F.FLINT_ERR_INVALID_ARG
    assert lib.flint_moe_create(layer, F.FLINT_MAX_LAYERS + 1, ctypes.byref(h)) == F.FLINT_ERR_INVALID_ARG
    assert lib.flint_moe_create(layer, 1, ctypes.byref(h)) == F.FLINT_ERR_INVALID_ARG   # null tensors
    assert "NULL" in F.flint_moe_last_error()
    assert lib.flint_moe_create(layer, 1, None) == F.FLINT_ERR_INVALID_ARG


def test_null_handle_calls():
    lib = F.lib()
    assert lib.flint_moe_forward(None, 16, 1, 0, 1, 16, None) == F.FLINT_ERR_INVALID_ARG
    assert lib.flint_moe_set_trace(None, None, None, 0) == F.FLINT_ERR_INVALID_ARG
    assert lib.flint_moe_status(None, None) == F.FLINT_ERR_INVALID_ARG
    lib.flint_moe_destroy(None)          # NULL-safe
    with pytest.raises(F.FlintMoEError):
        F.flint_moe_forward(None, 16, 1, 0, 1, 16)
