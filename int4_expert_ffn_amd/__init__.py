"""Python binding of libflint_moe.so, the MI355X library for the Flint MoE FFN
block.  Argument marshalling only: every step of the block runs in the HIP
kernels behind the C ABI declared in include/flint_moe.h.  PyTorch tensors are
accepted for convenience (their device pointers are passed through); raw
integer addresses work too.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# FLINT_MOE_LIBRARY selects another build of the same library (the profiling
# build with phase timestamps); by default the in-tree libflint_moe.so.
LIB_PATH = os.environ.get("FLINT_MOE_LIBRARY") or os.path.join(HERE, "libflint_moe.so")

FLINT_HIDDEN = 2048
FLINT_EXPERTS = 256
FLINT_EXPERT_SIZE = 512
FLINT_SHARED_SIZE = 1024
FLINT_TOP_K = 6
FLINT_GROUP = 128
FLINT_MAX_LAYERS = 64
FLINT_MAX_TOKENS = 2048
DECODE_MAX_TOKENS = 16

FLINT_OK = 0
FLINT_ERR_INVALID_ARG = -1
FLINT_ERR_OUT_OF_MEMORY = -2
FLINT_ERR_HIP = -3
FLINT_ERR_UNSUPPORTED = -4
FLINT_ERR_DEVICE = -5

FLINT_DENSE_MLP_SIZE = 6144
FLINT_VOCAB = 150144
FLINT_DENSE_MAX_TOKENS = 16

FLINT_ATT_Q_HEADS = 32
FLINT_ATT_KV_HEADS = 4
FLINT_ATT_HEAD_DIM = 128
FLINT_ATT_WINDOW = 513
FLINT_ATT_RING = 640
FLINT_ATT_MAX_TOKENS = 16
FLINT_ATT_SCRATCH_BYTES = 16 << 20

EXPORTED = ("flint_moe_create", "flint_moe_create_fp16_interm", "flint_moe_forward", "flint_moe_set_trace",
            "flint_moe_status", "flint_moe_debug_set_epoch", "flint_moe_debug_live_allocations",
            "flint_moe_destroy", "flint_moe_last_error", "flint_dense_mlp_forward",
            "flint_head_forward", "flint_attn_workspace_bytes", "flint_attn_decode", "flint_attn_decode_noalloc")


class flint_q4(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class flint_moe_layer(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("gate", flint_q4), ("up", flint_q4), ("down", flint_q4),
                ("sh_gate", flint_q4), ("sh_up", flint_q4), ("sh_down", flint_q4)]


class FlintMoEError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"flint_moe error {code}: {msg}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree library; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(f"{LIB_PATH} is missing: build it with int4_expert_ffn_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, ci = ctypes.c_void_p, ctypes.c_int
        L.flint_moe_create.argtypes = [ctypes.POINTER(flint_moe_layer), ci, ctypes.POINTER(vp)]
        L.flint_moe_create.restype = ci
        L.flint_moe_create_fp16_interm.argtypes = [ctypes.POINTER(flint_moe_layer), ci, ci, ctypes.POINTER(vp)]
        L.flint_moe_create_fp16_interm.restype = ci
        L.flint_moe_forward.argtypes = [vp, vp, ci, ci, ci, vp, vp]
        L.flint_moe_forward.restype = ci
        L.flint_moe_set_trace.argtypes = [vp, vp, vp, ci]
        L.flint_moe_set_trace.restype = ci
        L.flint_moe_status.argtypes = [vp, vp]
        L.flint_moe_status.restype = ci
        L.flint_moe_debug_set_epoch.argtypes = [vp, ctypes.c_uint32]
        L.flint_moe_debug_set_epoch.restype = ci
        L.flint_moe_debug_live_allocations.argtypes = []
        L.flint_moe_debug_live_allocations.restype = ci
        L.flint_moe_destroy.argtypes = [vp]
        L.flint_moe_destroy.restype = None
        L.flint_moe_last_error.argtypes = []
        L.flint_moe_last_error.restype = ctypes.c_char_p
        L.flint_dense_mlp_forward.argtypes = [flint_q4, flint_q4, flint_q4, ci, vp, ci, vp, vp, vp]
        L.flint_dense_mlp_forward.restype = ci
        L.flint_head_forward.argtypes = [flint_q4, ci, vp, ci, vp, vp]
        L.flint_head_forward.restype = ci
        L.flint_attn_workspace_bytes.argtypes = [ci, ci]
        L.flint_attn_workspace_bytes.restype = ctypes.c_size_t
        L.flint_attn_decode.argtypes = [vp, vp, vp, ci, vp, ctypes.POINTER(ctypes.c_int32), ci, ci, vp, vp,
                                        ctypes.c_size_t, vp]
        L.flint_attn_decode.restype = ci
        L.flint_attn_decode_noalloc.argtypes = [vp, vp, vp, ci, vp, ctypes.POINTER(ctypes.c_int32), ci, ci, vp, vp]
        L.flint_attn_decode_noalloc.restype = ci
        _lib = L
    return _lib


def _ptr(t) -> int:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _check(rc: int) -> int:
    if rc != FLINT_OK:
        raise FlintMoEError(rc, lib().flint_moe_last_error().decode())
    return rc


def layer_struct(d) -> flint_moe_layer:
    """Descriptor of one layer from a mapping with the canonical tensor names
    (router, bias, gate, gate_s, up, up_s, down, down_s, sh_gate, sh_gate_s,
    sh_up, sh_up_s, sh_down, sh_down_s)."""
    q = lambda c, s: flint_q4(_ptr(d[c]), _ptr(d[s]))
    return flint_moe_layer(_ptr(d["router"]), _ptr(d["bias"]), q("gate", "gate_s"), q("up", "up_s"),
                           q("down", "down_s"), q("sh_gate", "sh_gate_s"), q("sh_up", "sh_up_s"),
                           q("sh_down", "sh_down_s"))


def _layer_array(layers):
    return (flint_moe_layer * len(layers))(*[l if isinstance(l, flint_moe_layer) else layer_struct(l)
                                             for l in layers])


def flint_moe_create(layers) -> int:
    """layers: sequence of per-layer mappings (see layer_struct) or flint_moe_layer."""
    h = ctypes.c_void_p()
    _check(lib().flint_moe_create(_layer_array(layers), len(layers), ctypes.byref(h)))
    return h.value


def flint_moe_create_fp16_interm(layers, interm_div) -> int:
    """Handle for weights whose routed up projections are divided by
    ``interm_div``; SwiGLU outputs are rounded to fp16 (decode calls of up to 16 tokens)."""
    h = ctypes.c_void_p()
    _check(lib().flint_moe_create_fp16_interm(_layer_array(layers), len(layers), interm_div, ctypes.byref(h)))
    return h.value


def flint_moe_forward(h, x, n_tokens, layer_begin, layer_end, out, stream=None) -> None:
    _check(lib().flint_moe_forward(h, _ptr(x), n_tokens, layer_begin, layer_end, _ptr(out), _stream(stream)))


def flint_moe_set_trace(h, ids, weights, capacity) -> None:
    _check(lib().flint_moe_set_trace(h, _ptr(ids), _ptr(weights), capacity))


def flint_moe_status(h, stream=None) -> None:
    _check(lib().flint_moe_status(h, _stream(stream)))


def flint_moe_debug_set_epoch(h, epoch) -> None:
    _check(lib().flint_moe_debug_set_epoch(h, epoch))


def flint_moe_debug_live_allocations() -> int:
    return lib().flint_moe_debug_live_allocations()


def flint_moe_destroy(h) -> None:
    lib().flint_moe_destroy(h)


def flint_moe_last_error() -> str:
    return lib().flint_moe_last_error().decode()


def q4(codes, scales) -> flint_q4:
    """Descriptor of one int4 matrix (device tensors or addresses)."""
    return flint_q4(_ptr(codes), _ptr(scales))


def flint_dense_mlp_forward(gate, up, down, inter, x, n_tokens, h, out, stream=None) -> None:
    """gate, up, down: flint_q4 descriptors (see q4)."""
    _check(lib().flint_dense_mlp_forward(gate, up, down, inter, _ptr(x), n_tokens, _ptr(h), _ptr(out),
                                         _stream(stream)))


def flint_head_forward(head, rows, x, n_tokens, logits, stream=None) -> None:
    _check(lib().flint_head_forward(head, rows, _ptr(x), n_tokens, _ptr(logits), _stream(stream)))


def flint_attn_workspace_bytes(n_tokens, max_seen) -> int:
    return lib().flint_attn_workspace_bytes(n_tokens, max_seen)


def flint_attn_decode(q, k, v, ring_rows, sinks, pos, n_tokens, window, out, workspace, workspace_bytes,
                      stream=None) -> None:
    """pos: host sequence of n_tokens positions; the rest device tensors or addresses."""
    p = (ctypes.c_int32 * n_tokens)(*[int(x) for x in pos])
    _check(lib().flint_attn_decode(_ptr(q), _ptr(k), _ptr(v), ring_rows, _ptr(sinks), p, n_tokens, window, _ptr(out),
                                   _ptr(workspace), workspace_bytes, _stream(stream)))


def flint_attn_decode_noalloc(q, k, v, ring_rows, sinks, pos, n_tokens, window, out, stream=None) -> None:
    """flint_attn_decode with the library's fixed scratch instead of a workspace."""
    p = (ctypes.c_int32 * n_tokens)(*[int(x) for x in pos])
    _check(lib().flint_attn_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), ring_rows, _ptr(sinks), p, n_tokens, window,
                                           _ptr(out), _stream(stream)))


def _stream(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class FlintMoE:
    """Owning wrapper: ``FlintMoE(layers)``, ``forward(x, l0, l1, out)``.
    ``interm_div`` > 0 selects the fp16-intermediate form (see
    flint_moe_create_fp16_interm)."""

    def __init__(self, layers, interm_div=0):
        self.n_layers = len(layers)
        self.h = flint_moe_create_fp16_interm(layers, interm_div) if interm_div else flint_moe_create(layers)

    def forward(self, x, layer_begin=0, layer_end=None, out=None, stream=None):
        import torch
        if layer_end is None:
            layer_end = self.n_layers
        if out is None:
            out = torch.empty_like(x)
        if x.dtype != torch.float32 or not x.is_contiguous() or x.dim() != 2 or x.shape[1] != FLINT_HIDDEN:
            raise ValueError("x must be a contiguous float32 [n_tokens, 2048] tensor")
        flint_moe_forward(self.h, x, x.shape[0], layer_begin, layer_end, out, stream)
        return out

    def set_trace(self, ids, weights, capacity):
        flint_moe_set_trace(self.h, ids, weights, capacity)

    def status(self, stream=None):
        flint_moe_status(self.h, stream)

    def debug_set_epoch(self, epoch):
        flint_moe_debug_set_epoch(self.h, epoch)

    def close(self):
        if self.h:
            flint_moe_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
