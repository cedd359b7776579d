"""Pins of the oracle's decode attention with learned sinks (How to Run Flint
Locally, "Sinks and the 513-token window"; TandemLLM "21 Flint", 21.1 table).

- The page's own arithmetic for the sink: n window tokens tied at one logit s
  leave the sink 1 / (1 + n e^(s - o)) of the attention.
- With the sink pushed to -inf the layer is plain softmax attention, checked
  against PyTorch's scaled_dot_product_attention (a library routine).
- One visible position: out = v e^s / (e^s + e^o).
- Only the 513 positions ending at the token matter, wherever they sit in
  the ring.
- Query head h reads KV head h // 8.
"""
import math

import numpy as np
import torch

import flintgen as fg
from oracle import flint_oracle as O

HQ, HKV, D = fg.ATT_Q_HEADS, fg.ATT_KV_HEADS, fg.ATT_HEAD_DIM


def bf16_values(bits):
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).double().numpy()


def test_sink_share_closed_form():
    for n, s, o in [(1, 0.0, 0.0), (64, 1.5, 3.9), (513, -2.0, -9.0), (200, 4.0, 12.4), (7, 12.0, 0.5)]:
        q = np.zeros((HQ, D))
        q[:, 0] = s * math.sqrt(D)          # q . k / sqrt(D) = s for k = e_0
        k = np.zeros((n, HKV, D))
        k[:, :, 0] = 1.0
        v = np.zeros((n, HKV, D))
        v[:, :, 1] = 1.0
        out = O.attention_decode(q, k, v, np.full(HQ, o), pos=n - 1, window=0)
        share = 1.0 / (1.0 + n * math.exp(s - o))
        np.testing.assert_allclose(out[:, 1], 1.0 - share, rtol=1e-12, atol=1e-15)
        assert np.all(out[:, [0] + list(range(2, D))] == 0)


def test_without_sink_equals_library_attention():
    rng = np.random.default_rng(4)
    n = 300
    q = rng.standard_normal((HQ, D))
    k = rng.standard_normal((n, HKV, D))
    v = rng.standard_normal((n, HKV, D))
    out = O.attention_decode(q, k, v, np.full(HQ, -np.inf), pos=n - 1, window=0)
    kq = torch.from_numpy(np.repeat(k.transpose(1, 0, 2), HQ // HKV, axis=0))   # [HQ][n][D]
    vq = torch.from_numpy(np.repeat(v.transpose(1, 0, 2), HQ // HKV, axis=0))
    want = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q)[:, None, :], kq, vq)[:, 0, :]
    np.testing.assert_allclose(out, want.numpy(), rtol=1e-10, atol=1e-12)


def test_single_position_closed_form():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((HQ, D))
    k = rng.standard_normal((1, HKV, D))
    v = rng.standard_normal((1, HKV, D))
    sinks = rng.uniform(-9, 12.4, HQ)
    out = O.attention_decode(q, k, v, sinks, pos=0, window=513)
    for h in range(HQ):
        s = float(q[h] @ k[0, h // 8]) / math.sqrt(D)
        np.testing.assert_allclose(out[h], v[0, h // 8] * (1.0 / (1.0 + math.exp(sinks[h] - s))), rtol=1e-12)


def test_window_sees_513_positions_in_any_ring():
    """The token at position p sees p - 512 .. p; rows outside do not matter,
    and the same sequence held in a 640-row ring or a longer one gives the same
    output."""
    pos, W = 1500, fg.ATT_WINDOW
    rng = np.random.default_rng(6)
    seq_k = rng.standard_normal((pos + 1, HKV, D))
    seq_v = rng.standard_normal((pos + 1, HKV, D))
    q = rng.standard_normal((HQ, D))
    sinks = rng.uniform(-9, 12.4, HQ)
    full = O.attention_decode(q, seq_k, seq_v, sinks, pos, W)
    ring_k = np.zeros((fg.ATT_RING, HKV, D))
    ring_v = np.zeros((fg.ATT_RING, HKV, D))
    for p in range(pos + 1):            # write the sequence through the ring, oldest first
        ring_k[p % fg.ATT_RING] = seq_k[p]
        ring_v[p % fg.ATT_RING] = seq_v[p]
    assert np.array_equal(O.attention_decode(q, ring_k, ring_v, sinks, pos, W), full)
    seq_k2, seq_v2 = seq_k.copy(), seq_v.copy()
    seq_k2[: pos - W + 1] = rng.standard_normal((pos - W + 1, HKV, D))    # outside the window
    seq_v2[: pos - W + 1] = 0
    assert np.array_equal(O.attention_decode(q, seq_k2, seq_v2, sinks, pos, W), full)
    seq_v2[pos - W + 1] += 1.0                                           # the oldest position seen
    assert not np.array_equal(O.attention_decode(q, seq_k2, seq_v2, sinks, pos, W), full)


def test_query_heads_read_their_kv_group():
    rng = np.random.default_rng(7)
    n = 40
    q = rng.standard_normal((HQ, D))
    k = rng.standard_normal((n, HKV, D))
    for g in range(HKV):
        v = np.zeros((n, HKV, D))
        v[:, g] = rng.standard_normal((n, D))
        out = O.attention_decode(q, k, v, np.zeros(HQ), pos=n - 1, window=0)
        nz = np.flatnonzero(np.abs(out).sum(axis=1))
        assert nz.tolist() == list(range(8 * g, 8 * g + 8))


def test_generated_inputs_have_the_pages_shapes():
    q = fg.attn_queries(0, 0, 3)
    k, v = fg.attn_cache(0, 0, fg.ATT_RING)
    s = fg.attn_sinks(0, 0)
    assert q.shape == (3, 32, 128) and k.shape == v.shape == (640, 4, 128) and s.shape == (32,)
    assert -9.0 <= s.min() and s.max() <= 12.4
    assert np.array_equal(bf16_values(k).astype(np.float32).astype(np.float64), bf16_values(k))
