"""CPU oracle for the Flint per-token MoE FFN block.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call this module.  The GPU library never does: the
product path has no CPU fallback.

Plain, slow, obviously-correct NumPy in float64.  Every weight is dequantised
explicitly into a dense fp64 matrix, top-k is a full stable sort, and nothing is
blocked, fused or reordered beyond what the definition states.  It shares no
code with the HIP path.

What it computes, per token and per layer (sources are the pages' titles and
sections; see also the readings listed below):

* Residual recurrence x_{l+1} = x_l + moe_l(norm(x_l)) over the 47 MoE layers
  (How to Run Flint Locally, "The architecture, from config.json": layers 2..48
  are MoE layers).
* The block input is the RMS-normalised residual rounded to bf16 (weight-only
  W4A16 with bf16 activations: vLLM recipe "Flint", variants/nvfp4 entry and
  How to Run Flint Locally, "What vLLM changed"; the router is sensitive to one
  bf16 rounding of the residual: TandemLLM "21 Flint", section 21.1).
* Router: a sigmoid score per routed expert with a bias used for selection,
  top 6 of 256 kept and their weights normalised (How to Run Flint Locally,
  config table row "Routed experts" and the paragraph after the table;
  TandemLLM "21 Flint", 21.1 table row "MLP").
* Experts: SwiGLU FFN of gate/up matrices 512 x 2048 and down 2048 x 512; one
  shared expert of size 1,024 that runs for every token and is added beside
  the routed ones (same table rows "Routed experts", "Shared expert").
* Intermediates stay in high precision: the pages report SwiGLU activations
  near 2.6e5 in the top layers, past fp16 (TandemLLM "21 Flint", 21.2).

Readings taken where the pages are silent:
bias added after the sigmoid (c = s + b); routing weights from the unbiased s
of the picks, normalised to sum 1 with no epsilon and no extra scale; shared
expert added with weight 1; SiLU on the gate; exact ties in c go to the lower
expert index; RMSNorm epsilon 1e-6 and gain 1; symmetric int4 codes in
[-8, 7], byte j of a row holds k = 2j in bits 0-3 and k = 2j+1 in bits 4-7,
one bf16 scale per (row, group of G consecutive k).

Precision: all arithmetic in fp64; the two rounding points are the block input
(fp64 -> bf16, round to nearest even) and the residual after each layer
(fp64 -> fp32, round to nearest even), the interface dtypes.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

RMS_EPS = 1e-6


# ------------------------------------------------------------------ formats
def unpack_int4(codes) -> np.ndarray:
    """uint8 [..., K/2] -> int8 [..., K] of two's-complement 4-bit codes.

    Byte j holds element k = 2j in its low nibble and k = 2j + 1 in its high
    nibble; a nibble n stands for n when n < 8 and n - 16 otherwise.
    """
    c = np.asarray(codes).astype(np.uint8)
    lo = (c & 0x0F).astype(np.int16)
    hi = (c >> 4).astype(np.int16)
    v = np.empty(c.shape[:-1] + (2 * c.shape[-1],), dtype=np.int16)
    v[..., 0::2] = lo
    v[..., 1::2] = hi
    v = np.where(v >= 8, v - 16, v)
    return v.astype(np.int8)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (int16 or uint16) -> exact float64 values."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def dequant(codes, scale_bits, group: int) -> np.ndarray:
    """Dense fp64 matrix W[r, k] = code[r, k] * scale[r, k // group]."""
    v = unpack_int4(codes).astype(np.float64)
    s = bf16_bits_to_f64(scale_bits)
    if v.shape[-1] != s.shape[-1] * group:
        raise ValueError("scale groups do not cover K")
    return v * np.repeat(s, group, axis=-1)


def round_to_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value, ties to even (one rounding).

    bf16 keeps 8 significant bits and fp32's exponent range; below 2^-126 the
    spacing is fixed at 2^-133 (subnormals).
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                  # x = m * 2^e, 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)         # exponent of one unit in the last place
    y = np.ldexp(np.round(np.ldexp(x, -q)), q)   # np.round: half to even
    return np.where(x == 0, x, y)


def router_weights_f64(w) -> np.ndarray:
    """Router weights given as bf16 bits (int16/uint16) or fp32 values -> fp64."""
    w = np.asarray(w)
    if w.dtype in (np.int16, np.uint16):
        return bf16_bits_to_f64(w)
    if w.dtype == np.float32:
        return w.astype(np.float64)
    raise TypeError("router weights must be bf16 bits or float32")


# ------------------------------------------------------------------ pieces
def rms_normalise(x) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps), fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x) + RMS_EPS)


def sigmoid(z) -> np.ndarray:
    """1 / (1 + exp(-z)) in fp64, evaluated without overflow for either sign."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def silu(g) -> np.ndarray:
    return np.asarray(g, dtype=np.float64) * sigmoid(g)


@dataclasses.dataclass
class Route:
    z: np.ndarray          # router logits [E]
    s: np.ndarray          # sigmoid scores [E]
    c: np.ndarray          # selection scores s + b [E]
    order: np.ndarray      # all experts sorted by (-c, e)
    ids: np.ndarray        # chosen experts, in order
    weights: np.ndarray    # w_i = s_i / sum_T s
    margin: float          # c of the k-th pick minus c of the (k+1)-th


def route(a, router_w, bias, k: int, forced: Optional[Sequence[int]] = None) -> Route:
    """Sigmoid router with bias used for selection only.

    z = Wr a; s = sigmoid(z); c = s + b; the k experts with the largest c
    (ties to the lower index) are used, weighted by s normalised over the
    picks.  ``forced`` replaces the selection (its order is kept) while the
    weights are still the normalised s of the forced set.
    """
    wr = router_weights_f64(router_w)
    z = wr @ np.asarray(a, dtype=np.float64)
    s = sigmoid(z)
    c = s + np.asarray(bias, dtype=np.float32).astype(np.float64)
    e = np.arange(c.shape[0])
    order = np.lexsort((e, -c))         # primary -c, then index
    ids = order[:k] if forced is None else np.asarray(forced, dtype=np.int64)
    margin = float(c[order[k - 1]] - c[order[k]]) if k < c.shape[0] else float("inf")
    w = s[ids] / np.sum(s[ids])
    return Route(z=z, s=s, c=c, order=order, ids=ids, weights=w, margin=margin)


def swiglu_expert(wg, wu, wd, a):
    """y = Wd (silu(Wg a) * (Wu a)); returns (y, h) in fp64."""
    a = np.asarray(a, dtype=np.float64)
    g = wg @ a
    u = wu @ a
    h = silu(g) * u
    return wd @ h, h


# ------------------------------------------------------------------ block
@dataclasses.dataclass
class BlockResult:
    delta: np.ndarray      # sum_i w_i y_i + y_shared (fp64)
    route: Route
    max_abs_h: float       # largest |h| over the routed and shared experts


def _dense(src_ex, i, group):
    return (dequant(src_ex["gate"][i], src_ex["gate_s"][i], group),
            dequant(src_ex["up"][i], src_ex["up_s"][i], group),
            dequant(src_ex["down"][i], src_ex["down_s"][i], group))


def moe_block(a, src, layer: int, shape, forced=None) -> BlockResult:
    """One MoE block on the block input ``a`` (already normalised / rounded).

    ``src`` supplies the layer's tensors in the canonical layout: ``router(l)``,
    ``bias(l)``, ``experts(l, ids)`` (codes/scales of the listed routed
    experts) and ``shared(l)``.
    """
    r = route(a, src.router(layer), src.bias(layer), shape.top_k, forced)
    ex = src.experts(layer, [int(e) for e in r.ids])
    ex = {k: np.asarray(v) for k, v in ex.items()}
    delta = np.zeros(shape.hidden, dtype=np.float64)
    hmax = 0.0
    for i in range(len(r.ids)):
        wg, wu, wd = _dense(ex, i, shape.group)
        y, h = swiglu_expert(wg, wu, wd, a)
        delta += r.weights[i] * y
        hmax = max(hmax, float(np.max(np.abs(h))))
    sh = {k: np.asarray(v) for k, v in src.shared(layer).items()}
    y_sh, h_sh = swiglu_expert(dequant(sh["gate"], sh["gate_s"], shape.group),
                               dequant(sh["up"], sh["up_s"], shape.group),
                               dequant(sh["down"], sh["down_s"], shape.group), a)
    delta += y_sh
    hmax = max(hmax, float(np.max(np.abs(h_sh))))
    return BlockResult(delta=delta, route=r, max_abs_h=hmax)


# ------------------------------------------------------------------ fp16 intermediates
# TandemLLM "21 Flint", 21.2: in the last layers of the stack the routed
# experts' SwiGLU outputs grow to about 2.6e5, beyond fp16's largest value.
# The pack format therefore ships every routed up matrix scaled down by a
# power of two (expert_interm_div, 128 on that page) and scales the routing
# weights back up by it when the block runs.  Readings: the
# SwiGLU output of every expert, routed and shared, is rounded to fp16 before
# its down projection (round to nearest even, +-inf past the largest finite
# value); only the routed up projections are divided; gate and up are as in
# moe_block.


def round_to_fp16(x) -> np.ndarray:
    """fp64 -> the nearest fp16 value (ties to even; +-inf beyond the finite
    range), returned as fp64."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def moe_block_fp16_interm(a, src, layer: int, shape, interm_div: int, forced=None) -> BlockResult:
    """moe_block in the fp16-intermediate form.  ``src`` holds the pack's
    weights: every routed expert's up projection already divided by
    ``interm_div``.  max_abs_h is over the fp16 SwiGLU outputs."""
    r = route(a, src.router(layer), src.bias(layer), shape.top_k, forced)
    ex = src.experts(layer, [int(e) for e in r.ids])
    ex = {k: np.asarray(v) for k, v in ex.items()}
    a = np.asarray(a, dtype=np.float64)
    delta = np.zeros(shape.hidden, dtype=np.float64)
    hmax = 0.0
    for i in range(len(r.ids)):
        wg, wu, wd = _dense(ex, i, shape.group)
        h = round_to_fp16(silu(wg @ a) * (wu @ a))
        delta += (interm_div * r.weights[i]) * (wd @ h)
        hmax = max(hmax, float(np.max(np.abs(h))))
    sh = {k: np.asarray(v) for k, v in src.shared(layer).items()}
    g = dequant(sh["gate"], sh["gate_s"], shape.group) @ a
    u = dequant(sh["up"], sh["up_s"], shape.group) @ a
    h_sh = round_to_fp16(silu(g) * u)
    delta += dequant(sh["down"], sh["down_s"], shape.group) @ h_sh
    hmax = max(hmax, float(np.max(np.abs(h_sh))))
    return BlockResult(delta=delta, route=r, max_abs_h=hmax)


def block_input(x, shape) -> np.ndarray:
    """RMS-normalise the fp32 residual and round to bf16 (real shape)."""
    a = rms_normalise(np.asarray(x, dtype=np.float32).astype(np.float64))
    return round_to_bf16(a) if shape.act_bf16 else a


@dataclasses.dataclass
class LayerRecord:
    layer: int
    delta: np.ndarray
    route: Route
    max_abs_h: float
    x_out: np.ndarray      # fp32 residual after the layer


def moe_stack(x0, src, shape, layer_begin: int, layer_end: int,
              forced: Optional[dict] = None) -> List[LayerRecord]:
    """x_{l+1} = fp32(x_l + moe_l(bf16(rmsnorm(x_l)))) for l in [begin, end).

    ``forced`` maps a layer index to a selection that replaces the router's
    choice at that layer (used to continue after a near-tie).
    """
    x = np.asarray(x0, dtype=np.float32)
    recs = []
    for l in range(layer_begin, layer_end):
        a = block_input(x, shape)
        res = moe_block(a, src, l, shape, (forced or {}).get(l))
        x = (x.astype(np.float64) + res.delta).astype(np.float32)
        recs.append(LayerRecord(layer=l, delta=res.delta, route=res.route,
                                max_abs_h=res.max_abs_h, x_out=x))
    return recs


# ------------------------------------------------------------------ dense layers and head
# The model's other int4 matrix-vector products read per decode token (How to
# Run Flint Locally, "The architecture, from config.json": layers 0 and 1 have
# a dense MLP of size 6,144; "One decode step in bytes": every token reads the
# whole 150,144 x 2,048 output head, which the announcement quoted there keeps
# at 4 bits).  Readings: the dense MLP is the same SwiGLU as an expert, fed by
# the same block input (bf16 of the RMS-normalised residual) and added to the
# residual; the head is fed by the same normalisation and rounding of the final
# residual (epsilon 1e-6, gain 1), and its logits are fp64 here.

@dataclasses.dataclass
class DenseResult:
    delta: np.ndarray      # Wd h (fp64)
    h: np.ndarray          # silu(Wg a) * (Wu a) (fp64)
    x_out: np.ndarray      # fp32(x + delta)


def dense_mlp(x, w, shape) -> DenseResult:
    """x + Wd (silu(Wg a) * (Wu a)) with a = bf16(rmsnorm(x)); ``w`` holds
    gate/up codes [inter][H/2] and down codes [H][inter/2] with their scales."""
    a = block_input(x, shape)
    w = {k: np.asarray(v) for k, v in w.items()}
    y, h = swiglu_expert(dequant(w["gate"], w["gate_s"], shape.group),
                         dequant(w["up"], w["up_s"], shape.group),
                         dequant(w["down"], w["down_s"], shape.group), a)
    x_out = (np.asarray(x, dtype=np.float32).astype(np.float64) + y).astype(np.float32)
    return DenseResult(delta=y, h=h, x_out=x_out)


def head_logits(x, codes, scales, shape) -> np.ndarray:
    """logits[r] = sum_k W[r, k] a[k] in fp64 with a = bf16(rmsnorm(x)), for
    the rows given (codes [rows][H/2], scale bits [rows][H/G])."""
    a = block_input(x, shape)
    return dequant(np.asarray(codes), np.asarray(scales), shape.group) @ a


# ------------------------------------------------------------------ counts
def parameter_counts(shape, n_layers: int):
    """Per-token parameter counts read by one decode step of the MoE layers:
    routed (k experts x 3 matrices), shared (3 matrices of I_s), routers (E x H),
    summed over ``n_layers``; and per-expert / per-layer routed totals."""
    per_expert = 3 * shape.expert_size * shape.hidden
    return {
        "per_expert": per_expert,
        "per_layer_routed": shape.n_experts * per_expert,
        "all_layers_routed": n_layers * shape.n_experts * per_expert,
        "routed_per_token": n_layers * shape.top_k * per_expert,
        "shared_per_token": n_layers * 3 * shape.shared_size * shape.hidden,
        "router_per_token": n_layers * shape.n_experts * shape.hidden,
    }


def bytes_per_token_layer(shape, n_tokens_experts: int = None) -> int:
    """Algorithmic HBM bytes one token reads in one layer: bf16 router, fp32
    bias, and for each of the k routed experts plus the shared expert the
    int4 codes (K/2 bytes per row) and bf16 scales (K/G per row)."""
    def q4(rows, k):
        return rows * k // 2 + rows * (k // shape.group) * 2
    e = shape.top_k if n_tokens_experts is None else n_tokens_experts
    expert = 2 * q4(shape.expert_size, shape.hidden) + q4(shape.hidden, shape.expert_size)
    shared = 2 * q4(shape.shared_size, shape.hidden) + q4(shape.hidden, shape.shared_size)
    router = shape.n_experts * shape.hidden * 2 + shape.n_experts * 4
    return router + e * expert + shared


# ------------------------------------------------------------------ decode attention
# One layer's attention for one query token (How to Run Flint Locally, "Sinks
# and the 513-token window": a sliding layer attends over 513 positions, its own
# and the previous 512; a sink is one more softmax slot with a fixed logit, the head's
# learned offset, and no value vector.  TandemLLM "21 Flint", 21.1 table: query
# heads 32, KV heads 4, head size 128; window layers keep a ring of 640 rows; full
# layers see every position).  Readings: query head h reads KV head
# h // (32 / 4) (consecutive query heads share a KV head); scores are
# q . k / sqrt(128); the query, keys and values arrive already normed and
# rotated (this step does not include the projections, the QK norm or RoPE).


def attention_decode(q, k, v, sinks, pos: int, window: int, n_kv: int = 4) -> np.ndarray:
    """q [Hq][D] query values; k, v [R][n_kv][D] cache values with position p at
    row p % R; sinks [Hq]; the token at ``pos`` sees positions
    max(0, pos - window + 1) .. pos (window = 0: all of 0 .. pos).  Returns
    out [Hq][D] in fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, d = q.shape
    ring = k.shape[0]
    first = max(0, pos - window + 1) if window else 0
    if pos - first + 1 > ring:
        raise ValueError("the positions a token sees must fit the cache rows")
    rows = np.arange(first, pos + 1) % ring
    out = np.zeros((n_q, d))
    group = n_q // n_kv
    for h in range(n_q):
        g = h // group
        logits = np.concatenate([(k[rows, g, :] @ q[h]) / np.sqrt(d), [float(sinks[h])]])
        e = np.exp(logits - logits.max())
        p = e / e.sum()
        out[h] = p[:-1] @ v[rows, g, :]
    return out
