"""Pins of the oracle's dense-MLP and output-head functions (the model's other
int4 matrix-vector products: How to Run Flint Locally, "The architecture, from
config.json", table row "Dense MLP size"; "One decode step in bytes", the
output head).  Closed forms on one-hot weights, exact power-of-two scaling,
zero input, and a tiny case recomputed in 60-digit decimal arithmetic.
"""
import math
from decimal import Decimal, localcontext

import numpy as np
import pytest
import torch

import flintgen as fg
from oracle import flint_oracle as O
from oracle_sources import bf16_bits, pack_codes

FLINT = fg.FLINT
TINY = fg.TINY


def one_hot_q4(rows, K, G, r, k, v, rng):
    codes = np.zeros((rows, K), np.int64)
    codes[r, k] = v
    scales = bf16_bits(rng.uniform(0.005, 0.02, size=(rows, K // G)))
    return pack_codes(codes), scales, O.bf16_bits_to_f64(scales)[r, k // G]


def test_head_one_hot_closed_form():
    """One non-zero code v at (r, k) with scale sigma: logit r = v sigma a_k,
    every other logit 0, with a the bf16 block input of x."""
    rng = np.random.default_rng(11)
    x = fg.token(11, 0)
    a = O.block_input(x, FLINT)
    for (r, k, v) in [(0, 0, 7), (3, 2047, -8), (1, 130, -3), (4, 1, 5)]:
        codes, scales, sigma = one_hot_q4(5, FLINT.hidden, FLINT.group, r, k, v, rng)
        y = O.head_logits(x, codes, scales, FLINT)
        expect = np.zeros(5)
        expect[r] = v * sigma * a[k]
        assert np.array_equal(y, expect), (r, k, v)


def test_head_rows_are_independent_and_match_decimal():
    """Generated rows are the same whether taken alone or with the whole head,
    and each logit is the 60-digit decimal dot product within 1e-12."""
    rows = [0, 1, 77, fg.VOCAB - 1]
    c_sub, s_sub = fg.head(0, row_ids=rows)
    c_all, s_all = fg.head(0, rows=200)
    assert torch.equal(c_sub[:3], c_all[[0, 1, 77]]) and torch.equal(s_sub[:3], s_all[[0, 1, 77]])
    x = fg.token(0, 5)
    y = O.head_logits(x, c_sub.numpy(), s_sub.numpy(), FLINT)
    a = O.block_input(x, FLINT)
    sval = torch.tensor(s_sub.numpy()).view(torch.bfloat16).double().numpy()
    with localcontext() as ctx:
        ctx.prec = 60
        for i in range(len(rows)):
            acc = Decimal(0)
            for j, byte in enumerate(c_sub[i].numpy().tolist()):
                for half, n in enumerate((byte & 15, byte >> 4)):
                    kk = 2 * j + half
                    v = n - 16 if n >= 8 else n
                    acc += Decimal(v) * Decimal(float(sval[i, kk // FLINT.group])) * Decimal(float(a[kk]))
            assert abs(y[i] - float(acc)) <= 1e-12 * abs(float(acc)) + 1e-300, (i, y[i], acc)


def test_dense_mlp_one_hot_closed_form():
    """Gate and up one-hot in row i (at k1, k2), down one-hot at (r, i):
    delta_r = vd sd silu(vg sg a_k1) (vu su a_k2) and nothing else; SiLU on
    the up projection instead would give a different value."""
    rng = np.random.default_rng(12)
    H, inter, G = FLINT.hidden, 256, FLINT.group
    x = fg.token(12, 0)
    a = O.block_input(x, FLINT)
    i, k1, k2, r = 17, 5, 700, 1999
    gc, gs, sg = one_hot_q4(inter, H, G, i, k1, 6, rng)
    uc, us, su = one_hot_q4(inter, H, G, i, k2, -7, rng)
    dc, ds, sd = one_hot_q4(H, inter, G, r, i, 3, rng)
    res = O.dense_mlp(x, {"gate": gc, "gate_s": gs, "up": uc, "up_s": us, "down": dc, "down_s": ds}, FLINT)
    g, u = 6 * sg * a[k1], -7 * su * a[k2]
    h = g / (1 + math.exp(-g)) * u
    assert res.h[i] == pytest.approx(h, rel=1e-15) and np.count_nonzero(res.h) == 1
    assert res.delta[r] == pytest.approx(3 * sd * h, rel=1e-15) and np.count_nonzero(res.delta) == 1
    assert res.delta[r] != pytest.approx(3 * sd * u / (1 + math.exp(-u)) * g, rel=1e-6)
    assert np.array_equal(res.x_out, (x.astype(np.float64) + res.delta).astype(np.float32))


def _tiny_dense(seed):
    return fg.dense_layer(seed, 0, hidden=TINY.hidden, inter=128, group=TINY.group)


def test_dense_mlp_zero_input_and_power_of_two_scales():
    w = {k: v.numpy() for k, v in _tiny_dense(3).items()}
    z = O.dense_mlp(np.zeros(TINY.hidden, np.float32), w, TINY)
    assert np.all(z.delta == 0) and np.all(z.x_out == 0)
    x = fg.token(3, 1, TINY.hidden)
    base = O.dense_mlp(x, w, TINY)
    for j in (4, -3):
        wd = dict(w, down_s=(w["down_s"].astype(np.int32) + (j << 7)).astype(np.int16))
        assert np.array_equal(O.dense_mlp(x, wd, TINY).delta, base.delta * 2.0 ** j)
        wu = dict(w, up_s=(w["up_s"].astype(np.int32) + (j << 7)).astype(np.int16))
        r = O.dense_mlp(x, wu, TINY)
        assert np.array_equal(r.h, base.h * 2.0 ** j) and np.array_equal(r.delta, base.delta * 2.0 ** j)


def test_dense_mlp_against_decimal():
    """Tiny dense MLP (hidden 256, width 128, group 32, fp32 block input) in
    60-digit decimal arithmetic: fp64 oracle within 1e-12 relative."""
    w = {k: v.numpy() for k, v in _tiny_dense(4).items()}
    x = fg.token(4, 0, TINY.hidden)
    res = O.dense_mlp(x, w, TINY)
    a = O.block_input(x, TINY)
    with localcontext() as ctx:
        ctx.prec = 60
        D = Decimal

        def mv(codes, scales, vec):
            sv = torch.tensor(np.asarray(scales, np.int16)).view(torch.bfloat16).double().numpy()
            out = []
            for row in range(codes.shape[0]):
                acc = D(0)
                for j, byte in enumerate(codes[row].tolist()):
                    for half, n in enumerate((byte & 15, byte >> 4)):
                        k = 2 * j + half
                        acc += D(n - 16 if n >= 8 else n) * D(float(sv[row, k // TINY.group])) * vec[k]
                out.append(acc)
            return out

        av = [D(float(v)) for v in a]
        g = mv(w["gate"], w["gate_s"], av)
        u = mv(w["up"], w["up_s"], av)
        h = [gg / (D(1) + (-gg).exp()) * uu for gg, uu in zip(g, u)]
        y = mv(w["down"], w["down_s"], h)
        ref = np.array([float(v) for v in y])
    assert np.max(np.abs(res.delta - ref)) <= 1e-12 * np.max(np.abs(ref))
