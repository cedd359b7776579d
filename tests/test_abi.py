"""The C-ABI library: it loads, exports every function include/*.h declares,
and rejects invalid arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import int4_expert_ffn_amd as F

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADER = os.path.join(INCLUDE, "flint_moe.h")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))


def declared_functions():
    names = set()
    for hdr in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(hdr).read(), flags=re.S)
        names |= set(re.findall(r"\b(flint_\w+)\s*\(", text))
    return sorted(names)


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
    text = open(os.path.join(INCLUDE, "flint_dense.h")).read()
    for name in ("FLINT_DENSE_MLP_SIZE", "FLINT_VOCAB", "FLINT_DENSE_MAX_TOKENS"):
        m = re.search(r"#define\s+%s\s+(-?\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(F, name), name
    text = open(os.path.join(INCLUDE, "flint_attn.h")).read()
    for name in ("FLINT_ATT_Q_HEADS", "FLINT_ATT_KV_HEADS", "FLINT_ATT_HEAD_DIM", "FLINT_ATT_WINDOW", "FLINT_ATT_RING",
                 "FLINT_ATT_MAX_TOKENS"):
        m = re.search(r"#define\s+%s\s+(-?\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(F, name), name


def test_attention_rejects_bad_arguments_before_any_hip_call():
    lib = F.lib()
    A = 16   # any non-null, 16-byte aligned address: validation fails before it is used
    ws = F.flint_attn_workspace_bytes(1, 513)
    assert ws == 1 * 32 * 9 * 132 * 4     # 9 chunks of 64 positions, 132 floats per head
    assert F.flint_attn_workspace_bytes(1, 768) == 1 * 32 * 12 * 132 * 4
    assert F.flint_attn_workspace_bytes(2, 769) == 2 * 32 * 12 * 132 * 4   # 4 chunks of 256, or 12 of 64 for others
    assert F.flint_attn_workspace_bytes(1, 100000) == 1 * 32 * 391 * 132 * 4
    assert F.flint_attn_workspace_bytes(0, 513) == 0 and F.flint_attn_workspace_bytes(17, 513) == 0
    assert F.flint_attn_workspace_bytes(1, 0) == 0
    inval = F.FLINT_ERR_INVALID_ARG

    def call(pos, n=None, window=513, ring=640, q=A, out=1 << 20, wsb=ws, ws_ptr=1 << 21):
        n = len(pos) if n is None else n
        p = (ctypes.c_int32 * max(1, len(pos)))(*pos)
        return lib.flint_attn_decode(q, A, A, ring, A, p, n, window, out, ws_ptr, wsb, None)

    assert call([10], n=0) == inval
    assert call([10] * 17) == inval
    assert call([-1]) == inval
    assert call([10], ring=0) == inval
    assert call([10], window=-1) == inval
    assert call([700], window=0) == inval                  # 701 positions, 640 rows
    assert call([5000], wsb=ws - 1) == inval               # window 513 fits the ring; workspace too small
    assert call([10], q=A + 4) == inval                    # misaligned
    assert call([10], out=A) == inval                      # out overlaps q
    assert "overlaps" in F.flint_moe_last_error()
    assert lib.flint_attn_decode(None, A, A, 640, A, (ctypes.c_int32 * 1)(3), 1, 513, A, A, ws, None) == inval
    # the allocation-free variant: the same checks, and its scratch limit
    def call_na(pos, n=None, window=513, ring=640, q=A, out=1 << 20):
        n = len(pos) if n is None else n
        p = (ctypes.c_int32 * max(1, len(pos)))(*pos)
        return lib.flint_attn_decode_noalloc(q, A, A, ring, A, p, n, window, out, None)

    assert call_na([10], n=0) == inval
    assert call_na([-1]) == inval
    assert call_na([700], window=0) == inval
    assert call_na([10], out=A) == inval
    assert call_na([15872] * 16, window=0, ring=16000) == inval   # 16 x 63 chunks: above the 16 MiB scratch
    assert "scratch" in F.flint_moe_last_error()
    assert call_na([253952], window=0, ring=300000) == inval       # one token, 993 chunks
    assert F.flint_attn_workspace_bytes(1, 253952) <= F.FLINT_ATT_SCRATCH_BYTES
    assert F.flint_attn_workspace_bytes(16, 15872) <= F.FLINT_ATT_SCRATCH_BYTES


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
    for div in (-128, 3, 96, 1 << 16):   # the fp16-intermediate divisor: a power of two in [1, 32768]
        h = ctypes.c_void_p(1234)
        assert lib.flint_moe_create_fp16_interm(layer, 1, div, ctypes.byref(h)) == F.FLINT_ERR_INVALID_ARG
        assert h.value is None
        assert "interm_div" in F.flint_moe_last_error()
    assert lib.flint_moe_create_fp16_interm(layer, 1, 128, ctypes.byref(h)) == F.FLINT_ERR_INVALID_ARG  # null tensors


def test_null_handle_calls():
    lib = F.lib()
    assert lib.flint_moe_forward(None, 16, 1, 0, 1, 16, None) == F.FLINT_ERR_INVALID_ARG
    assert lib.flint_moe_set_trace(None, None, None, 0) == F.FLINT_ERR_INVALID_ARG
    assert lib.flint_moe_status(None, None) == F.FLINT_ERR_INVALID_ARG
    lib.flint_moe_destroy(None)          # NULL-safe
    with pytest.raises(F.FlintMoEError):
        F.flint_moe_forward(None, 16, 1, 0, 1, 16)


def test_dense_and_head_reject_bad_arguments_before_any_hip_call():
    """Fake but aligned addresses: every call fails validation, so nothing is
    enqueued and no GPU is needed."""
    lib = F.lib()
    A = 1 << 20
    good = F.q4(A, A)
    inval = F.FLINT_ERR_INVALID_ARG
    H, W = F.FLINT_HIDDEN, F.FLINT_DENSE_MLP_SIZE
    x, h, out = 16 * A, 32 * A, 48 * A
    # dense MLP
    assert lib.flint_dense_mlp_forward(F.q4(None, A), good, good, W, x, 1, h, out, None) == inval
    assert lib.flint_dense_mlp_forward(F.q4(A + 8, A), good, good, W, x, 1, h, out, None) == inval
    assert lib.flint_dense_mlp_forward(F.q4(A, A + 2), good, good, W, x, 1, h, out, None) == inval
    assert lib.flint_dense_mlp_forward(good, good, good, W, None, 1, h, out, None) == inval
    assert lib.flint_dense_mlp_forward(good, good, good, W, x + 4, 1, h, out, None) == inval
    for n in (0, F.FLINT_DENSE_MAX_TOKENS + 1):
        assert lib.flint_dense_mlp_forward(good, good, good, W, x, n, h, out, None) == inval
    for inter in (0, 1024, 3000, W + 2048):
        assert lib.flint_dense_mlp_forward(good, good, good, inter, x, 1, h, out, None) == inval
    assert lib.flint_dense_mlp_forward(good, good, good, W, x, 2, h, x + 16 * 4, None) == inval   # partial overlap
    assert lib.flint_dense_mlp_forward(good, good, good, W, x, 1, x + 4 * H - 16, x, None) == inval   # h overlaps
    assert "overlap" in F.flint_moe_last_error()
    # head
    assert lib.flint_head_forward(F.q4(A, None), 10, x, 1, out, None) == inval
    assert lib.flint_head_forward(good, 0, x, 1, out, None) == inval
    assert lib.flint_head_forward(good, 10, x, 0, out, None) == inval
    assert lib.flint_head_forward(good, 10, x, 17, out, None) == inval
    assert lib.flint_head_forward(good, 10, x + 8, 1, out, None) == inval
    assert lib.flint_head_forward(good, 10, x, 1, x + 64, None) == inval
    with pytest.raises(F.FlintMoEError):
        F.flint_head_forward(good, 0, x, 1, out)
