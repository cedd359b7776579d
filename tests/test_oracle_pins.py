"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, swapped nibbles, the wrong matrix
under SiLU, weights from biased scores) fails at least one of them.
"""
import itertools
import json
import math
import os
from decimal import Decimal, localcontext

import numpy as np
import pytest
import scipy.special
import torch

import flintgen as fg
from oracle import flint_oracle as O
from oracle_sources import ArraySource, SynthSource, bf16_bits, pack_codes, synth_source

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TINY = fg.TINY
FLINT = fg.FLINT


# ------------------------------------------------------------ formats
def test_unpack_nibble_order_and_sign():
    # byte 0x7F: k=0 <- low nibble 0xF = -1, k=1 <- high nibble 0x7 = 7
    assert O.unpack_int4(np.array([[0x7F, 0x80, 0x08, 0x00]], np.uint8)).tolist() == \
        [[-1, 7, 0, -8, -8, 0, 0, 0]]
    rng = np.random.default_rng(5)
    v = rng.integers(-8, 8, size=(7, 64))
    assert np.array_equal(O.unpack_int4(pack_codes(v)), v)


def test_bf16_decode_and_rounding_match_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 16, size=4000).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]          # finite only
    ref = torch.tensor(bits.astype(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(O.bf16_bits_to_f64(bits), ref)
    # fp32 inputs, including exact ties (bf16 value + half an ulp) and subnormals
    x = np.concatenate([rng.standard_normal(5000), rng.standard_normal(500) * 1e-38,
                        rng.standard_normal(500) * 1e30]).astype(np.float32)
    b = O.bf16_bits_to_f64(bits[:2000])
    ties = (b + np.ldexp(1.0, np.frexp(b)[1] - 9)).astype(np.float32)   # exactly half-way
    x = np.concatenate([x, ties, -ties])
    want = torch.tensor(x).to(torch.bfloat16).double().numpy()
    got = O.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_rounding_of_fp64_is_single_rounding():
    # 1 + 2^-8 + 2^-40 is just above the midpoint between 1 and 1 + 2^-7: a
    # single rounding gives 1 + 2^-7; rounding through fp32 first would give 1.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert O.round_to_bf16(np.array([x]))[0] == 1.0 + 2.0 ** -7
    assert O.round_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0          # tie -> even
    assert O.round_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


def test_dequant_one_hot_closed_form():
    """A single non-zero code v at (r, k) with scale sigma gives (W a)[r] = v sigma a_k."""
    rng = np.random.default_rng(2)
    rows, K, G = 6, 256, 32
    a = rng.standard_normal(K)
    for (r, k, v) in [(0, 0, 7), (1, 1, -8), (2, 31, 3), (3, 32, -1), (5, 255, 5), (4, 100, -6)]:
        codes = np.zeros((rows, K), np.int64)
        codes[r, k] = v
        scales = bf16_bits(rng.uniform(0.005, 0.02, size=(rows, K // G)))
        sigma = O.bf16_bits_to_f64(scales)[r, k // G]
        W = O.dequant(pack_codes(codes), scales, G)
        y = W @ a
        expect = np.zeros(rows)
        expect[r] = v * sigma * a[k]
        assert np.array_equal(y, expect), (r, k, v)


# ------------------------------------------------------------ pieces
def test_sigmoid_matches_library_and_symmetry():
    z = np.concatenate([np.linspace(-40, 40, 2001), [-800.0, 800.0, 0.0]])
    s = O.sigmoid(z)
    assert np.allclose(s, scipy.special.expit(z), rtol=1e-15, atol=0)
    assert np.allclose(s + O.sigmoid(-z), 1.0, rtol=0, atol=1e-15)
    assert O.sigmoid(np.array([0.0]))[0] == 0.5


def test_rmsnorm_closed_forms():
    x = np.full(2048, 3.0)
    assert np.allclose(O.rms_normalise(x), 1.0 / math.sqrt(1 + O.RMS_EPS / 9.0), rtol=1e-15)
    assert np.all(O.rms_normalise(np.zeros(16)) == 0)
    rng = np.random.default_rng(3)
    v = rng.standard_normal(2048) * 50
    # scale invariance (up to the epsilon term)
    assert np.allclose(O.rms_normalise(v), O.rms_normalise(4 * v), rtol=1e-9)
    assert abs(np.mean(O.rms_normalise(v) ** 2) - 1) < 1e-8


def test_swiglu_silu_on_gate_closed_form():
    """g = 2, u = 3 from one-hot matrices -> h = 6 sigmoid(2); swapping gate and
    up would give 6 sigmoid(3)."""
    I, K = 4, 8
    a = np.zeros(K)
    a[0] = 1.0
    wg = np.zeros((I, K)); wg[0, 0] = 2.0
    wu = np.zeros((I, K)); wu[0, 0] = 3.0
    wd = np.zeros((K, I)); wd[5, 0] = 1.0
    y, h = O.swiglu_expert(wg, wu, wd, a)
    assert h[0] == pytest.approx(6.0 / (1.0 + math.exp(-2.0)), rel=1e-15)
    assert h[0] != pytest.approx(6.0 / (1.0 + math.exp(-3.0)), rel=1e-6)
    assert y[5] == h[0] and np.count_nonzero(y) == 1


# ------------------------------------------------------------ selection
def _route_with_scores(z, b, k):
    """Drive O.route with a one-hot block input so that z is exactly chosen."""
    E = len(z)
    wr = np.zeros((E, 4), np.float32)
    wr[:, 0] = np.asarray(z, np.float32)
    a = np.array([1.0, 0, 0, 0])
    return O.route(a, wr, np.asarray(b, np.float32), k)


@pytest.mark.parametrize("E,k,seed", [(16, 2, 0), (16, 2, 1), (24, 6, 2)])
def test_topk_equals_bruteforce_best_subset(E, k, seed):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(E).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    r = _route_with_scores(z, b, k)
    best = max(itertools.combinations(range(E), k), key=lambda S: sum(r.c[list(S)]))
    assert sorted(r.ids.tolist()) == sorted(best)
    # ids are listed by decreasing c, and the margin is the k-th minus the (k+1)-th
    assert np.all(np.diff(r.c[r.ids]) <= 0)
    rest = np.setdiff1d(np.arange(E), r.ids)
    assert r.margin == pytest.approx(r.c[r.ids].min() - r.c[rest].max(), abs=0)


def test_topk_exact_ties_go_to_lower_index():
    z = np.array([0.5, 1.0, 1.0, 1.0, -2.0], np.float32)
    b = np.zeros(5, np.float32)
    r = _route_with_scores(z, b, 2)
    assert r.ids.tolist() == [1, 2] and r.margin == 0.0


def test_weights_use_unbiased_scores():
    z = np.array([0.0, 1.0, -1.0, 2.0], np.float32)
    b = np.array([0.9, 0.0, 0.8, -0.5], np.float32)   # changes the ranking
    r = _route_with_scores(z, b, 2)
    s = scipy.special.expit(z.astype(np.float64))
    c = s + b.astype(np.float64)
    top = sorted(range(4), key=lambda e: (-c[e], e))[:2]
    assert r.ids.tolist() == top
    assert np.allclose(r.weights, s[top] / s[top].sum(), rtol=1e-15)
    assert r.weights.sum() == pytest.approx(1.0, abs=1e-15)


# ------------------------------------------------------------ exact arithmetic
def test_block_against_high_precision_decimal():
    """Tiny block recomputed in 60-digit decimal arithmetic from the same codes:
    fp64 oracle within 1e-12 relative."""
    src = synth_source(TINY, seed=0)
    x = fg.token(0, 0, TINY.hidden)
    res = O.moe_block(x.astype(np.float64), src, 0, TINY)
    with localcontext() as ctx:
        ctx.prec = 60
        D = Decimal
        a = [D(float(v)) for v in x]

        def deq(codes, scales, G):
            sval = torch.tensor(np.asarray(scales, np.int16)).view(torch.bfloat16).double().numpy()
            out = []
            for r in range(codes.shape[0]):
                row = []
                for j in range(codes.shape[1]):
                    byte = int(codes[r, j])
                    for half, n in enumerate((byte & 15, byte >> 4)):
                        k = 2 * j + half
                        v = n - 16 if n >= 8 else n
                        row.append(D(v) * D(float(sval[r, k // G])))
                out.append(row)
            return out

        def mv(W, v):
            return [sum((w * x_ for w, x_ in zip(row, v)), D(0)) for row in W]

        def sig(t):
            return D(1) / (D(1) + (-t).exp())

        wr = [[D(float(w)) for w in row] for row in np.asarray(src.router(0), np.float32)]
        b = [D(float(v)) for v in src.bias(0)]
        z = mv(wr, a)
        s = [sig(t) for t in z]
        c = [s[e] + b[e] for e in range(len(s))]
        T = sorted(range(len(c)), key=lambda e: (-c[e], e))[:TINY.top_k]
        assert T == res.route.ids.tolist()
        tot = sum((s[e] for e in T), D(0))
        delta = [D(0)] * TINY.hidden
        ex = src.experts(0, T)
        for i, e in enumerate(T):
            g = mv(deq(ex["gate"][i], ex["gate_s"][i], TINY.group), a)
            u = mv(deq(ex["up"][i], ex["up_s"][i], TINY.group), a)
            h = [gg * sig(gg) * uu for gg, uu in zip(g, u)]
            y = mv(deq(ex["down"][i], ex["down_s"][i], TINY.group), h)
            delta = [d + (s[e] / tot) * yy for d, yy in zip(delta, y)]
        sh = src.shared(0)
        g = mv(deq(sh["gate"], sh["gate_s"], TINY.group), a)
        u = mv(deq(sh["up"], sh["up_s"], TINY.group), a)
        h = [gg * sig(gg) * uu for gg, uu in zip(g, u)]
        y = mv(deq(sh["down"], sh["down_s"], TINY.group), h)
        delta = [d + yy for d, yy in zip(delta, y)]
        ref = np.array([float(d) for d in delta])
    err = np.max(np.abs(res.delta - ref)) / np.max(np.abs(ref))
    assert err < 1e-12, err


# ------------------------------------------------------------ invariants
def test_zero_input_gives_zero_and_bias_topk():
    src = synth_source(TINY, seed=1)
    res = O.moe_block(np.zeros(TINY.hidden), src, 0, TINY)
    assert np.all(res.delta == 0)
    b = src.bias(0).astype(np.float64)
    assert res.route.ids.tolist() == sorted(range(TINY.n_experts), key=lambda e: (-b[e], e))[:TINY.top_k]
    assert np.all(res.route.s == 0.5)
    # stack at the real shape: x = 0 stays 0 through normalisation and layers
    ssrc = SynthSource(fg.Synth(FLINT, 0, 2))
    recs = O.moe_stack(np.zeros(FLINT.hidden, np.float32), ssrc, FLINT, 0, 2)
    assert all(np.all(r.x_out == 0) for r in recs)


def _identical_experts(src: ArraySource, which=0):
    ex = {k: np.repeat(v[which:which + 1], v.shape[0], axis=0) for k, v in src.ex.items()}
    return src.replace(experts=ex)


def test_identical_experts_make_output_independent_of_routing():
    base = _identical_experts(synth_source(TINY, seed=2))
    x = fg.token(2, 0, TINY.hidden).astype(np.float64)
    r1 = O.moe_block(x, base, 0, TINY)
    other = synth_source(TINY, seed=3)
    r2 = O.moe_block(x, base.replace(router=other.router(0), bias=other.bias(0)), 0, TINY)
    assert r1.route.ids.tolist() != r2.route.ids.tolist()
    assert np.allclose(r1.delta, r2.delta, rtol=1e-13, atol=1e-13 * np.abs(r1.delta).max())
    # equals one expert plus the shared expert
    ex0 = {k: v[0] for k, v in base.ex.items()}
    y, _ = O.swiglu_expert(O.dequant(ex0["gate"], ex0["gate_s"], TINY.group),
                           O.dequant(ex0["up"], ex0["up_s"], TINY.group),
                           O.dequant(ex0["down"], ex0["down_s"], TINY.group), x)
    sh = base.sh
    ysh, _ = O.swiglu_expert(O.dequant(sh["gate"], sh["gate_s"], TINY.group),
                             O.dequant(sh["up"], sh["up_s"], TINY.group),
                             O.dequant(sh["down"], sh["down_s"], TINY.group), x)
    assert np.allclose(r1.delta, y + ysh, rtol=1e-13, atol=1e-13 * np.abs(ysh).max())


def test_exactly_k_routed_plus_shared_channels():
    """Routed expert e writes only output row e and the shared expert only row
    E: exactly k + 1 non-zero channels, with routed values in the ratio of the
    unbiased scores (closed form)."""
    shape = TINY
    src = _identical_experts(synth_source(shape, seed=4))
    E, H = shape.n_experts, shape.hidden
    down = src.ex["down"].copy()
    row = down[0, 7].copy()
    row[row == 0] = 0x11                      # make the kept row surely non-zero
    down[:] = 0
    down_s = src.ex["down_s"].copy()
    for e in range(E):
        down[e, e] = row
        down_s[e, e] = src.ex["down_s"][0, 7]   # same row content and scales for every expert
    sh = dict(src.sh)
    shd = np.zeros_like(sh["down"])
    shd[E] = 0x23
    sh["down"] = shd
    src = src.replace(experts=dict(src.ex, down=down, down_s=down_s), shared=sh)
    x = fg.token(4, 1, H).astype(np.float64)
    res = O.moe_block(x, src, 0, shape)
    nz = set(np.flatnonzero(res.delta).tolist())
    assert nz == set(res.route.ids.tolist()) | {E}
    vals = res.delta[res.route.ids]
    s = res.route.s[res.route.ids]
    assert np.allclose(vals / vals.sum(), s / s.sum(), rtol=1e-12)


def test_bias_affects_selection_only():
    src = synth_source(TINY, seed=5)
    E = TINY.n_experts
    pick = [3, 11]
    b = np.full(E, -10.0, np.float32)
    b[pick] = 10.0
    x = fg.token(5, 0, TINY.hidden).astype(np.float64)
    r1 = O.moe_block(x, src.replace(bias=b), 0, TINY)
    r2 = O.moe_block(x, src.replace(bias=2 * b), 0, TINY)
    r3 = O.moe_block(x, src, 0, TINY, forced=sorted(pick, key=lambda e: -r1.route.c[e]))
    assert sorted(r1.route.ids.tolist()) == pick
    assert np.array_equal(r1.delta, r2.delta)
    assert np.allclose(r1.delta, r3.delta, rtol=1e-15, atol=1e-15 * np.abs(r1.delta).max())


def test_power_of_two_scales_scale_output_exactly():
    src = synth_source(TINY, seed=6)
    x = fg.token(6, 0, TINY.hidden).astype(np.float64)
    base = O.moe_block(x, src, 0, TINY)
    for j in (3, -2):
        ex = dict(src.ex, down_s=(src.ex["down_s"].astype(np.int32) + (j << 7)).astype(np.int16))
        sh = dict(src.sh, down_s=(src.sh["down_s"].astype(np.int32) + (j << 7)).astype(np.int16))
        r = O.moe_block(x, src.replace(experts=ex, shared=sh), 0, TINY)
        assert np.array_equal(r.delta, base.delta * 2.0 ** j)
        ex = dict(src.ex, up_s=(src.ex["up_s"].astype(np.int32) + (j << 7)).astype(np.int16))
        sh = dict(src.sh, up_s=(src.sh["up_s"].astype(np.int32) + (j << 7)).astype(np.int16))
        r = O.moe_block(x, src.replace(experts=ex, shared=sh), 0, TINY)
        assert np.array_equal(r.delta, base.delta * 2.0 ** j)
        assert r.max_abs_h == base.max_abs_h * 2.0 ** j


def test_permutation_equivariance():
    src = synth_source(TINY, seed=7)
    E = TINY.n_experts
    perm = np.random.default_rng(7).permutation(E)       # new expert i is old perm[i]
    ex = {k: v[perm] for k, v in src.ex.items()}
    psrc = src.replace(router=src.router(0)[perm], bias=src.bias(0)[perm], experts=ex)
    x = fg.token(7, 0, TINY.hidden).astype(np.float64)
    r0 = O.moe_block(x, src, 0, TINY)
    r1 = O.moe_block(x, psrc, 0, TINY)
    assert r0.route.margin > 1e-9
    assert perm[r1.route.ids].tolist() == r0.route.ids.tolist()
    assert np.allclose(r0.delta, r1.delta, rtol=1e-13, atol=1e-13 * np.abs(r0.delta).max())


def test_fp32_range_needed_with_scaled_up_projection():
    """With up scales x 4096 at the real shape, SwiGLU intermediates pass
    fp16's largest finite value (65504) and stay finite in the oracle, while
    the same products in float16 overflow."""
    synth = fg.Synth(FLINT, 0, 1, up_scale_mult={0: 4096})
    src = SynthSource(synth)
    x = fg.token(0, 3)
    a = O.block_input(x, FLINT)
    res = O.moe_block(a, src, 0, FLINT)
    assert 65504 < res.max_abs_h < 1e7 and np.all(np.isfinite(res.delta))
    ex = src.experts(0, res.route.ids)
    hmax, worst = 0.0, None
    for i in range(len(res.route.ids)):
        g = O.dequant(ex["gate"][i], ex["gate_s"][i], FLINT.group) @ a
        u = O.dequant(ex["up"][i], ex["up_s"][i], FLINT.group) @ a
        h = O.silu(g) * u
        if np.max(np.abs(h)) > hmax:
            hmax, worst = float(np.max(np.abs(h))), (g, u)
    assert hmax > 65504
    g, u = worst
    with np.errstate(over="ignore"):
        h16 = (g.astype(np.float16) * O.sigmoid(g).astype(np.float16)) * u.astype(np.float16)
    assert np.isinf(h16).any()


def test_stack_layer_range_composes():
    ssrc = SynthSource(fg.Synth(FLINT, 0, 3))
    x = fg.token(0, 9)
    full = O.moe_stack(x, ssrc, FLINT, 0, 3)
    first = O.moe_stack(x, ssrc, FLINT, 0, 1)
    rest = O.moe_stack(first[-1].x_out, ssrc, FLINT, 1, 3)
    assert np.array_equal(full[-1].x_out, rest[-1].x_out)
    assert full[-1].x_out.dtype == np.float32


# ------------------------------------------------------------ the pages' counts
def test_parameter_counts_match_the_pages():
    with open(os.path.join(GOLDEN, "flint_param_counts.json")) as f:
        gold = {e["name"]: e for e in json.load(f)["entries"]}
    c = O.parameter_counts(FLINT, fg.N_LAYERS_FLINT)

    def check(name, value):
        e = gold[name]
        assert round(value / e["unit"]) * e["unit"] == pytest.approx(e["printed"], rel=1e-12), (name, value)

    for name in ("per_expert", "per_layer_routed", "all_layers_routed", "routed_per_token",
                 "shared_per_token", "router_per_token"):
        check(name, c[name])
    H = FLINT.hidden
    attention = 49 * (H * 4096 + 2 * H * 512 + 4096 * H)
    dense = 2 * 3 * H * fg.DENSE_MLP_SIZE
    check("attention_total", attention)
    check("dense_mlp_total", dense)
    moe = c["routed_per_token"] + c["shared_per_token"] + c["router_per_token"]
    rest = gold["body_total"]["printed"] - attention - dense - moe
    check("norms_and_sinks", rest)
    assert fg.VOCAB * H == gold["lm_head"]["printed"]
    assert gold["body_total"]["printed"] + gold["lm_head"]["printed"] == gold["active_total"]["printed"]
    # bytes one token reads per layer in this build's int4 format
    assert O.bytes_per_token_layer(FLINT) == 14_025_728
