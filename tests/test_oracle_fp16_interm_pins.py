"""Pins of the oracle's fp16-intermediate form (TandemLLM "21 Flint", 21.2: the
packs divide each routed expert's up projection by expert_interm_div so SwiGLU
outputs fit fp16, with the factor restored through the routing weights).

The form differs from the fp32 block only by one rounding of each SwiGLU
output to fp16.  Round to nearest even moves a value v in fp16's normal range
by at most 2^-11 |v|, and one in the subnormal range by at most 2^-25, so each
output element of the two forms differs by at most

    B[n] = sum_i d w_i sum_j |Wd_i[n, j]| (2^-11 |h_ij| / d + 2^-25)
         + sum_j |Wd_sh[n, j]| (2^-11 |h_sh,j| + 2^-25)

with h the fp32 form's SwiGLU outputs and d the divisor.  A dropped or doubled
divisor, a rounding put on the wrong value (y instead of h) or to the wrong
format (bf16: 2^-9), or no rounding at all fails one of these pins.
"""
import numpy as np

import flintgen as fg
from oracle import flint_oracle as O
from oracle_sources import SynthSource, synth_source

TINY = fg.TINY
FLINT = fg.FLINT


def test_round_to_fp16_closed_forms():
    cases = {
        1.0 + 2.0 ** -11: 1.0,                           # tie -> even (1.0)
        1.0 + 3 * 2.0 ** -11: 1.0 + 2.0 ** -9,           # tie -> even mantissa
        1.0 + 2.0 ** -11 + 2.0 ** -40: 1.0 + 2.0 ** -10,  # just above the tie: one rounding from fp64
        -(1.0 + 2.0 ** -11 + 2.0 ** -40): -(1.0 + 2.0 ** -10),
        65504.0: 65504.0,                                # largest finite
        65519.99: 65504.0,
        65520.0: np.inf,                                 # tie between 65504 and 2^16 -> even -> overflow
        -65520.0: -np.inf,
        2.0 ** -24: 2.0 ** -24,                          # smallest subnormal
        2.0 ** -25: 0.0,                                 # tie -> even (0)
        1.5 * 2.0 ** -25: 2.0 ** -24,
        3 * 2.0 ** -25: 2.0 ** -23,                      # tie between 1 and 2 subnormal ulps -> even
    }
    x = np.array(list(cases.keys()))
    want = np.array(list(cases.values()))
    got = O.round_to_fp16(x)
    assert np.array_equal(got, want), list(zip(x, got, want))


def _bound_and_delta(a, std_src, layer, shape, div, route):
    """The fp32 form's delta and the bound B above, from plain fp64 dense algebra."""
    ex = std_src.experts(layer, [int(e) for e in route.ids])
    delta = np.zeros(shape.hidden)
    bound = np.zeros(shape.hidden)
    for i in range(len(route.ids)):
        wg = O.dequant(ex["gate"][i], ex["gate_s"][i], shape.group)
        wu = O.dequant(ex["up"][i], ex["up_s"][i], shape.group)
        wd = O.dequant(ex["down"][i], ex["down_s"][i], shape.group)
        y, h = O.swiglu_expert(wg, wu, wd, a)
        delta += route.weights[i] * y
        bound += div * route.weights[i] * (np.abs(wd) @ (2.0 ** -11 * np.abs(h) / div + 2.0 ** -25))
    sh = std_src.shared(layer)
    wd = O.dequant(sh["down"], sh["down_s"], shape.group)
    y, h = O.swiglu_expert(O.dequant(sh["gate"], sh["gate_s"], shape.group),
                           O.dequant(sh["up"], sh["up_s"], shape.group), wd, a)
    delta += y
    bound += np.abs(wd) @ (2.0 ** -11 * np.abs(h) + 2.0 ** -25)
    return delta, bound


def _check_form(std_src, pack_src, layer, shape, div, x, rel_max=2e-3):
    a = O.block_input(x, shape)
    res = O.moe_block_fp16_interm(a, pack_src, layer, shape, div)
    ref = O.moe_block(a, std_src, layer, shape)
    assert res.route.ids.tolist() == ref.route.ids.tolist()      # the router is untouched
    delta, bound = _bound_and_delta(a, std_src, layer, shape, div, ref.route)
    np.testing.assert_allclose(delta, ref.delta, rtol=1e-12, atol=1e-300)
    diff = np.abs(res.delta - ref.delta)
    assert np.all(diff <= bound * (1 + 1e-9) + 1e-12 * np.abs(ref.delta)), float(np.max(diff / bound))
    rel = np.linalg.norm(res.delta - ref.delta) / np.linalg.norm(ref.delta)
    # the rounding is really there: well above fp64 noise, and of fp16's size
    assert 1e-6 < rel < rel_max, rel
    return rel, res


def test_fp16_form_within_rounding_bound_tiny():
    for seed in range(4):
        std = synth_source(TINY, seed=seed)
        pack = synth_source(TINY, seed=seed, up_scale_div=128)
        for t in range(3):
            _check_form(std, pack, 0, TINY, 128, fg.token(seed, t, TINY.hidden))


def test_fp16_form_within_rounding_bound_flint_shape():
    std = SynthSource(fg.Synth(FLINT, seed=0, n_layers=1))
    pack = SynthSource(fg.Synth(FLINT, seed=0, n_layers=1, up_scale_div=128))
    # Round-to-nearest errors have an rms of at most 2^-11 / sqrt(3) of |h|
    # (about 2.8e-4); over 2,048 outputs the relative L2 error stays near that,
    # and 6e-4 allows twice it.  bf16 rounding (2^-9 / sqrt(3)) would not fit.
    rel, res = _check_form(std, pack, 0, FLINT, 128, fg.token(0, 5), rel_max=6e-4)
    print(f"fp16-intermediate vs fp32 form: rel-L2 {rel:.2e}, max |h| {res.max_abs_h:.3g}")


def test_divisor_keeps_scaled_layer_finite():
    """A layer whose routed up scales are x4096 (the top layers of the stack):
    SwiGLU outputs pass fp16's range.  Without the divisor the fp16 form
    overflows; with the pack's /128 it stays finite and within the bound."""
    std = SynthSource(fg.Synth(FLINT, seed=7, n_layers=1, up_scale_mult={0: 4096}))
    pack = SynthSource(fg.Synth(FLINT, seed=7, n_layers=1, up_scale_mult={0: 4096}, up_scale_div=128))
    x = fg.token(7, 0)
    a = O.block_input(x, FLINT)
    raw = O.moe_block_fp16_interm(a, std, 0, FLINT, 1)
    assert not np.all(np.isfinite(raw.delta))
    assert O.moe_block(a, std, 0, FLINT).max_abs_h > 65504.0
    rel, res = _check_form(std, pack, 0, FLINT, 128, x)
    assert np.all(np.isfinite(res.delta)) and res.max_abs_h < 65504.0
