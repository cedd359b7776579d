"""Seeded synthetic inputs for the Flint MoE FFN block.

This package only draws numbers: weights (int4 codes and bf16 scales), router
weights and biases, and residual-stream tokens. It holds none of the block's
arithmetic (no dequantisation, no products, no routing). The CPU oracle's tests
and the GPU library's tests and benchmark both take their inputs from here, so
the two sides see the same bytes without sharing any computation.

Shapes follow the pages: hidden 2,048, 256 routed experts of size 512, top-6,
one shared expert of size 1,024, 47 MoE layers (How to Run Flint Locally,
"The architecture, from config.json", table rows "Hidden size", "Routed
experts", "Shared expert", "Layers").  The int4 format (symmetric codes in
[-8, 7], two per byte along K, bf16 scale per row and K-group) and the value
distributions are the synthetic workload's own choices: the pages publish no
weights here.

Bulk tensors use a counter-based generator so that any single expert can be
regenerated on its own (the oracle needs only the experts a token picks) and
whole layers can be generated on the GPU: every 32-bit word is
``lowbias32(lowbias32((i + k1) mod 2^32) xor k2)`` where ``i`` counts words in
one (layer, tensor, expert) block and ``(k1, k2)`` are derived from the block's
key.  ``lowbias32`` is Chris Wellons' published 32-bit integer hash
(xorshift-multiply, constants 0x7feb352d and 0x846ca68b).
Small tensors (router weights, biases, tokens) use NumPy's PCG64 streams keyed
by ``SeedSequence``.
"""
from __future__ import annotations

import dataclasses
from fractions import Fraction
from functools import lru_cache
from typing import Dict, Optional

import numpy as np
import torch

MASK32 = 0xFFFFFFFF

# tensor ids used in block keys
T_GATE, T_UP, T_DOWN = 0, 1, 2
T_GATE_S, T_UP_S, T_DOWN_S = 3, 4, 5
T_SH_GATE, T_SH_UP, T_SH_DOWN = 6, 7, 8
T_SH_GATE_S, T_SH_UP_S, T_SH_DOWN_S = 9, 10, 11
T_ROUTER, T_BIAS = 12, 13
# the model's other int4 matrices: the dense MLP of layers 0 and 1, the head
T_DENSE_GATE, T_DENSE_UP, T_DENSE_DOWN = 14, 15, 16
T_DENSE_GATE_S, T_DENSE_UP_S, T_DENSE_DOWN_S = 17, 18, 19
T_HEAD, T_HEAD_S = 20, 21
# decode attention inputs
T_ATT_Q, T_ATT_K, T_ATT_V, T_ATT_SINK = 22, 23, 24, 25
TOKEN_BASE = 1_000_000
DENSE_MLP_SIZE = 6144   # config table row "Dense MLP size" (layers 0 and 1)
VOCAB = 150144          # config table row "Vocabulary": rows of the output head


@dataclasses.dataclass(frozen=True)
class Shape:
    """Dimensions of one MoE block (names follow the pages' config table)."""
    hidden: int          # H
    n_experts: int       # E routed experts per layer
    expert_size: int     # I
    shared_size: int     # I_s
    top_k: int           # k
    group: int           # G, K-group of one bf16 scale
    router_bf16: bool    # router weights stored as bf16 (real shape) or fp32 (tiny)
    act_bf16: bool       # block input rounded to bf16 after RMSNorm


FLINT = Shape(hidden=2048, n_experts=256, expert_size=512, shared_size=1024,
              top_k=6, group=128, router_bf16=True, act_bf16=True)
TINY = Shape(hidden=256, n_experts=16, expert_size=64, shared_size=128,
             top_k=2, group=32, router_bf16=False, act_bf16=False)
N_LAYERS_FLINT = 47


# ---------------------------------------------------------------- hashing
def lowbias32_int(x: int) -> int:
    """Scalar reference of the hash (plain Python ints)."""
    x &= MASK32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & MASK32
    x ^= x >> 15
    x = (x * 0x846CA68B) & MASK32
    x ^= x >> 16
    return x


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2^32 for int64 tensors holding values in [0, 2^32), no int64 overflow."""
    lo = (x & 0xFFFF) * c
    hi = ((x >> 16) * c) & 0xFFFF
    return (lo + (hi << 16)) & MASK32


def lowbias32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def block_key(seed: int, layer: int, tensor: int, expert: int):
    h = 0x6A09E667
    for v in (seed, layer, tensor, expert):
        h = lowbias32_int(h ^ (v & MASK32))
    return h, lowbias32_int(h ^ 0x5BE0CD19)


def words_int(seed: int, layer: int, tensor: int, expert: int, i: int) -> int:
    """Scalar reference: word ``i`` of one block."""
    k1, k2 = block_key(seed, layer, tensor, expert)
    return lowbias32_int(lowbias32_int((i + k1) & MASK32) ^ k2)


def _words(keys, n: int, device) -> torch.Tensor:
    """Words [len(keys)][n] (int64 holding uint32) for a list of (k1, k2) keys."""
    k1 = torch.tensor([k[0] for k in keys], dtype=torch.int64, device=device)[:, None]
    k2 = torch.tensor([k[1] for k in keys], dtype=torch.int64, device=device)[:, None]
    i = torch.arange(n, dtype=torch.int64, device=device)[None, :]
    return lowbias32(lowbias32((i + k1) & MASK32) ^ k2)


def _words_at(key, idx: torch.Tensor) -> torch.Tensor:
    """Words at the given indices (int64 tensor) of one block."""
    k1, k2 = key
    return lowbias32(lowbias32((idx + k1) & MASK32) ^ k2)


def _words_to_bytes(w: torch.Tensor) -> torch.Tensor:
    """Little-endian bytes of uint32 words held in int64: [..., n] -> uint8 [..., 4n]."""
    w32 = torch.where(w >= 2 ** 31, w - 2 ** 32, w).to(torch.int32)
    return w32.contiguous().view(torch.uint8)


# ---------------------------------------------------------------- scales
SCALE_LO = Fraction(1, 200)   # 0.005
SCALE_HI = Fraction(1, 50)    # 0.02


def bf16_bits_value(bits: int) -> Fraction:
    """Exact value of a positive finite normal bf16 bit pattern."""
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    return Fraction(128 + m, 128) * (Fraction(2) ** (e - 127))


@lru_cache(maxsize=None)
def scale_table():
    """Integer table mapping a 24-bit draw m to bf16 bits of RNE(U(0.005, 0.02)).

    The uniform draw is u = (m + 1/2) / 2^24; the value 0.005 + 0.015 u is
    rounded to the nearest bf16 (ties to even mantissa), exactly, with
    rationals.  Returns (thresholds, bits): the bf16 bits for m are
    ``bits[#{t in thresholds : t <= m}]``.
    """
    def val(m):
        return SCALE_LO + (SCALE_HI - SCALE_LO) * Fraction(2 * m + 1, 2 ** 25)

    cands = [b for b in range(0x3B00, 0x3D00)]
    cands = [b for b in cands if Fraction(1, 400) <= bf16_bits_value(b) <= Fraction(1, 25)]

    def rne(v):
        best = None
        for b in cands:
            d = abs(bf16_bits_value(b) - v)
            if best is None or d < best[0] or (d == best[0] and (b & 1) == 0):
                best = (d, b)
        return best[1]

    lo_b, hi_b = rne(val(0)), rne(val(2 ** 24 - 1))
    bits = [b for b in cands if lo_b <= b <= hi_b]
    thresholds = []
    for j in range(1, len(bits)):
        mu = (bf16_bits_value(bits[j - 1]) + bf16_bits_value(bits[j])) / 2
        # smallest m whose value rounds to bits[j]
        q = (mu - SCALE_LO) / (SCALE_HI - SCALE_LO) * 2 ** 24 - Fraction(1, 2)
        m = int(q // 1)
        if val(m) < mu or (val(m) == mu and (bits[j] & 1)):
            m += 1
        while m > 0 and rne(val(m - 1)) == bits[j]:
            m -= 1
        while rne(val(m)) != bits[j]:
            m += 1
        thresholds.append(m)
    return thresholds, bits


def _scales_from_words(w: torch.Tensor) -> torch.Tensor:
    thr, bits = scale_table()
    t = torch.tensor(thr, dtype=torch.int64, device=w.device)
    b = torch.tensor(bits, dtype=torch.int64, device=w.device)
    idx = torch.bucketize(w >> 8, t, right=True)
    return b[idx].to(torch.int16)


# ---------------------------------------------------------------- generator
@dataclasses.dataclass
class Synth:
    """Seeded synthetic weights for a stack of MoE layers.

    ``up_scale_mult`` maps a layer index to a power-of-two multiplier of the
    routed experts' up-projection scales (exact in bf16); ``up_scale_div``
    divides them in every layer by a power of two (the fp16-intermediate pack
    form).  ``bias_kind`` is
    "uniform" (U(-0.1, 0.1)) or "zipf" (b_e = -0.05 * 1.1 * ln r_e, r a seeded
    permutation of 1..E).
    """
    shape: Shape = FLINT
    seed: int = 0
    n_layers: int = 1
    up_scale_mult: Optional[Dict[int, int]] = None
    bias_kind: str = "uniform"
    up_scale_div: int = 1

    # -- int4 code blocks
    def _codes(self, layer, tensor, experts, rows, k, device):
        n_words = rows * k // 8
        keys = [block_key(self.seed, layer, tensor, e) for e in experts]
        w = _words(keys, n_words, device)
        return _words_to_bytes(w).reshape(len(experts), rows, k // 2)

    def _scales(self, layer, tensor, experts, rows, k, device):
        ng = k // self.shape.group
        keys = [block_key(self.seed, layer, tensor, e) for e in experts]
        w = _words(keys, rows * ng, device)
        return _scales_from_words(w).reshape(len(experts), rows, ng)

    def _up_shift(self, layer):
        mult = (self.up_scale_mult or {}).get(layer, 1)
        sh = int(mult).bit_length() - 1
        dsh = int(self.up_scale_div).bit_length() - 1
        if mult != 1 << sh or self.up_scale_div != 1 << dsh:
            raise ValueError("up-scale multiplier and divisor must be powers of two")
        return sh - dsh

    def experts(self, layer: int, experts, device="cpu"):
        """Codes/scales of the given routed experts: dict of uint8/int16 tensors
        gate/up codes [n][I][H/2], scales [n][I][H/G]; down codes [n][H][I/2],
        scales [n][H][I/G]."""
        s = self.shape
        experts = list(experts)
        out = {
            "gate": self._codes(layer, T_GATE, experts, s.expert_size, s.hidden, device),
            "up": self._codes(layer, T_UP, experts, s.expert_size, s.hidden, device),
            "down": self._codes(layer, T_DOWN, experts, s.hidden, s.expert_size, device),
            "gate_s": self._scales(layer, T_GATE_S, experts, s.expert_size, s.hidden, device),
            "up_s": self._scales(layer, T_UP_S, experts, s.expert_size, s.hidden, device),
            "down_s": self._scales(layer, T_DOWN_S, experts, s.hidden, s.expert_size, device),
        }
        sh = self._up_shift(layer)
        if sh:
            out["up_s"] = out["up_s"] + (sh << 7)  # exponent field + sh: exact x 2^sh (scales are normal, positive)
        return out

    def shared(self, layer: int, device="cpu"):
        """Shared expert: gate/up codes [I_s][H/2], scales [I_s][H/G];
        down codes [H][I_s/2], scales [H][I_s/G]."""
        s = self.shape
        f = lambda t, r, k: self._codes(layer, t, [0], r, k, device)[0]
        g = lambda t, r, k: self._scales(layer, t, [0], r, k, device)[0]
        return {
            "gate": f(T_SH_GATE, s.shared_size, s.hidden),
            "up": f(T_SH_UP, s.shared_size, s.hidden),
            "down": f(T_SH_DOWN, s.hidden, s.shared_size),
            "gate_s": g(T_SH_GATE_S, s.shared_size, s.hidden),
            "up_s": g(T_SH_UP_S, s.shared_size, s.hidden),
            "down_s": g(T_SH_DOWN_S, s.hidden, s.shared_size),
        }

    def router(self, layer: int) -> torch.Tensor:
        """Router weights [E][H]: N(0, 1/H); bf16 bits (int16) for the real
        shape, float32 for the tiny one."""
        s = self.shape
        rng = np.random.default_rng(np.random.SeedSequence([self.seed, layer, T_ROUTER, 0]))
        w = (rng.standard_normal((s.n_experts, s.hidden)) / np.sqrt(s.hidden)).astype(np.float32)
        t = torch.from_numpy(w)
        return t.to(torch.bfloat16).view(torch.int16) if s.router_bf16 else t

    def bias(self, layer: int) -> torch.Tensor:
        s = self.shape
        rng = np.random.default_rng(np.random.SeedSequence([self.seed, layer, T_BIAS, 0]))
        if self.bias_kind == "uniform":
            b = rng.uniform(-0.1, 0.1, s.n_experts)
        elif self.bias_kind == "zipf":
            r = rng.permutation(s.n_experts) + 1
            b = -0.05 * 1.1 * np.log(r)
        else:
            raise ValueError(self.bias_kind)
        return torch.from_numpy(b.astype(np.float32))

    def layer(self, layer: int, device="cpu"):
        """Every tensor of one layer in the canonical layout (experts contiguous,
        expert-major), on ``device``."""
        ex = self.experts(layer, range(self.shape.n_experts), device)
        sh = self.shared(layer, device)
        out = {k: v for k, v in ex.items()}
        out.update({"sh_" + k: v for k, v in sh.items()})
        out["router"] = self.router(layer).to(device)
        out["bias"] = self.bias(layer).to(device)
        return out


def q4_matrix(seed: int, layer: int, tensor: int, scale_tensor: int, rows: int, k: int, group: int = 128,
              device="cpu", row_ids=None):
    """One int4 matrix [rows][k] of the same distributions as the experts:
    codes uint8 [r][k/2] and bf16 scale bits int16 [r][k/group].  ``row_ids``
    (a sequence of row indices) generates only those rows; each row's bytes
    do not depend on which other rows are generated."""
    wc, ws = k // 8, k // group
    kc = block_key(seed, layer, tensor, 0)
    ks = block_key(seed, layer, scale_tensor, 0)
    if row_ids is None:
        codes = _words_to_bytes(_words([kc], rows * wc, device)).reshape(rows, k // 2)
        scales = _scales_from_words(_words([ks], rows * ws, device)).reshape(rows, ws)
        return codes, scales
    r = torch.as_tensor(list(row_ids), dtype=torch.int64, device=device)[:, None]
    if bool(((r < 0) | (r >= rows)).any()):
        raise ValueError("row index out of range")
    codes = _words_to_bytes(_words_at(kc, r * wc + torch.arange(wc, device=device)[None, :]))
    scales = _scales_from_words(_words_at(ks, r * ws + torch.arange(ws, device=device)[None, :]))
    return codes.reshape(len(r), k // 2), scales.reshape(len(r), ws)


def dense_layer(seed: int, layer: int, device="cpu", hidden: int = FLINT.hidden, inter: int = DENSE_MLP_SIZE,
                group: int = 128):
    """Dense SwiGLU MLP of model layer 0 or 1: gate/up codes [inter][hidden/2],
    scales [inter][hidden/G]; down codes [hidden][inter/2], scales [hidden][inter/G]."""
    g = q4_matrix(seed, layer, T_DENSE_GATE, T_DENSE_GATE_S, inter, hidden, group, device)
    u = q4_matrix(seed, layer, T_DENSE_UP, T_DENSE_UP_S, inter, hidden, group, device)
    d = q4_matrix(seed, layer, T_DENSE_DOWN, T_DENSE_DOWN_S, hidden, inter, group, device)
    return {"gate": g[0], "gate_s": g[1], "up": u[0], "up_s": u[1], "down": d[0], "down_s": d[1]}


def head(seed: int, device="cpu", rows: int = VOCAB, hidden: int = FLINT.hidden, group: int = 128, row_ids=None):
    """Output head [rows][hidden] int4: (codes, scale bits); ``row_ids`` as in q4_matrix."""
    return q4_matrix(seed, 0, T_HEAD, T_HEAD_S, rows, hidden, group, device, row_ids)


def token(seed: int, t: int, hidden: int = FLINT.hidden) -> np.ndarray:
    """Residual-stream token t: x ~ N(0, 1) in float32."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, TOKEN_BASE + t]))
    return rng.standard_normal(hidden).astype(np.float32)


def tokens(seed: int, idx, hidden: int = FLINT.hidden) -> np.ndarray:
    return np.stack([token(seed, int(t), hidden) for t in idx])


def flint_stack(seed: int = 0, n_layers: int = N_LAYERS_FLINT, mult: int = 4096, up_div: int = 1) -> Synth:
    """The 47-layer stack workload: the last ten layers (37..46) multiply the
    routed up-projection scales by ``mult`` so SwiGLU intermediates reach the
    1e5 range the pages report for the top layers.  ``up_div`` > 1 gives the
    fp16-intermediate pack form of the same weights (routed up scales divided
    by it in every layer)."""
    top = {l: mult for l in range(max(0, n_layers - 10), n_layers)} if n_layers == N_LAYERS_FLINT else {}
    return Synth(FLINT, seed, n_layers, up_scale_mult=top, up_scale_div=up_div)


# ---------------------------------------------------------------- decode attention
# Attention of one layer (TandemLLM "21 Flint", 21.1 table rows "attention",
# "sliding layers", "full layers"; How to Run Flint Locally, "Sinks and the
# 513-token window"): query heads 32, KV heads 4, head size 128, a 513-position window
# held in a ring of 640 rows on window layers, every position on full layers,
# one learned sink logit per query head (the checkpoint's offsets run from -9.0
# to 12.4).
ATT_Q_HEADS, ATT_KV_HEADS, ATT_HEAD_DIM = 32, 4, 128
ATT_WINDOW, ATT_RING = 513, 640


def attn_queries(seed: int, layer: int, n_tokens: int) -> np.ndarray:
    """q [n][32][128] fp32, N(0, 1) per element (as after the per-head RMS norm)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, layer, T_ATT_Q, n_tokens]))
    return rng.standard_normal((n_tokens, ATT_Q_HEADS, ATT_HEAD_DIM)).astype(np.float32)


def attn_cache(seed: int, layer: int, rows: int):
    """k, v caches [rows][4][128] as bf16 bit patterns (int16), N(0, 1) values."""
    out = []
    for t in (T_ATT_K, T_ATT_V):
        rng = np.random.default_rng(np.random.SeedSequence([seed, layer, t, rows]))
        x = torch.from_numpy(rng.standard_normal((rows, ATT_KV_HEADS, ATT_HEAD_DIM), dtype=np.float32))
        out.append(x.to(torch.bfloat16).view(torch.int16).numpy())
    return out[0], out[1]


def attn_sinks(seed: int, layer: int) -> np.ndarray:
    """One sink logit per query head: U(-9.0, 12.4) rounded to bf16, as fp32."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, layer, T_ATT_SINK, 0]))
    x = torch.from_numpy(rng.uniform(-9.0, 12.4, ATT_Q_HEADS).astype(np.float32))
    return x.to(torch.bfloat16).float().numpy()
