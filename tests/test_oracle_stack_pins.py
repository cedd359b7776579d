"""Pins of the oracle's layer recurrence and of its block input rounding.

The stack is x_{l+1} = x_l + moe_l(rmsnorm(x_l)) over the MoE layers (How to
Run Flint Locally, "The architecture, from config.json": the MoE layers sit on
the residual stream), with the residual kept in fp32 between layers.  The
block input is the normalised residual rounded once to bf16 (TandemLLM "21
Flint", 21.1: a single bf16 rounding of the residual changes which experts the
router picks).  Every expected value below is written out by hand or follows
from an exact construction, not from the function under test.
"""
from fractions import Fraction

import numpy as np

import flintgen as fg
from oracle import flint_oracle as O
from oracle_sources import SynthSource

FLINT = fg.FLINT
TINY = fg.TINY


class ZeroExperts:
    """A layer source whose experts (routed and shared) are all-zero codes:
    every block output is exactly zero whatever the routing.  Router and bias
    come from the seeded generator, so the routing itself is ordinary."""

    def __init__(self, shape, seed=0, n_layers=3):
        self.shape = shape
        self.s = fg.Synth(shape, seed, n_layers)

    def router(self, layer):
        return self.s.router(layer).numpy()

    def bias(self, layer):
        return self.s.bias(layer).numpy()

    def _q(self, rows, k):
        return np.zeros((rows, k // 2), np.uint8), np.full((rows, k // self.shape.group), 0x3C00, np.int16)

    def experts(self, layer, ids):
        sh, n = self.shape, len(list(ids))
        gc, gs = self._q(sh.expert_size, sh.hidden)
        dc, ds = self._q(sh.hidden, sh.expert_size)
        rep = lambda a: np.repeat(a[None], n, axis=0)
        return {"gate": rep(gc), "gate_s": rep(gs), "up": rep(gc), "up_s": rep(gs),
                "down": rep(dc), "down_s": rep(ds)}

    def shared(self, layer):
        sh = self.shape
        gc, gs = self._q(sh.shared_size, sh.hidden)
        dc, ds = self._q(sh.hidden, sh.shared_size)
        return {"gate": gc, "gate_s": gs, "up": gc, "up_s": gs, "down": dc, "down_s": ds}


def test_stack_with_zero_blocks_keeps_the_residual_exactly():
    """Blocks that add nothing leave every layer's output equal to its input,
    bit for bit (a recurrence that dropped the residual would return 0)."""
    for shape in (TINY, FLINT):
        x0 = fg.token(0, 3, shape.hidden).astype(np.float32) * np.float32(3.0)
        recs = O.moe_stack(x0, ZeroExperts(shape), shape, 0, 3)
        assert len(recs) == 3
        for r in recs:
            assert np.all(r.delta == 0.0)
            assert r.x_out.dtype == np.float32
            assert np.array_equal(r.x_out, x0)


def test_stack_is_the_fp32_residual_recurrence():
    """Two layers equal fp32(fp32(x0 + d0) + d1), with each layer's block
    output d taken on the block input of that layer's own input."""
    src = SynthSource(fg.Synth(FLINT, 0, 2))
    x0 = fg.token(0, 21)
    recs = O.moe_stack(x0, src, FLINT, 0, 2)
    d0 = O.moe_block(O.block_input(x0, FLINT), src, 0, FLINT).delta
    x1 = (x0.astype(np.float64) + d0).astype(np.float32)
    d1 = O.moe_block(O.block_input(x1, FLINT), src, 1, FLINT).delta
    x2 = (x1.astype(np.float64) + d1).astype(np.float32)
    assert np.array_equal(recs[0].x_out, x1)
    assert np.array_equal(recs[1].x_out, x2)
    assert np.array_equal(recs[1].delta, d1)
    assert not np.array_equal(x1, x0) and not np.array_equal(x1, d0.astype(np.float32))


# ---------------------------------------------------------------- block input
# Residual of integers m with sum(m^2) = 2^51 exactly, so mean(x^2) = 2^40 and
# 1e-6 vanishes in its fp64 sum: the normalised value is exactly m * 2^-20, and
# the bf16 rounding of crafted m lands on or next to rounding midpoints.
P = 2 ** 20
SPECIAL = [  # (m, bf16 bits of the nearest bf16 to m / 2^20, ties to even)
    (P + 2 ** 12, 0x3F80),           # 1 + 2^-8: midpoint of 1 and 1 + 2^-7 -> even 1
    (P + 3 * 2 ** 12, 0x3F82),       # 1 + 3 2^-8: midpoint -> even 1 + 2^-6
    (P + 2 ** 12 + 1, 0x3F81),       # just above the first midpoint -> 1 + 2^-7
    (P + 2 ** 12 - 1, 0x3F80),       # just below it -> 1
    (-(P + 3 * 2 ** 12), 0xBF82),    # negative midpoint -> -(1 + 2^-6)
    (-(P + 2 ** 12 + 1), 0xBF81),
    (2 ** 19 + 2 ** 11, 0x3F00),     # 0.5 + 2^-9: midpoint of 0.5 and 0.5 + 2^-8 -> 0.5
    (2 ** 19 + 3 * 2 ** 11, 0x3F02),  # 0.5 + 3 2^-9: midpoint -> 0.5 + 2^-7
    (2 ** 21 - 2 ** 12, 0x4000),     # 2 - 2^-8: midpoint of 2 - 2^-7 and 2 -> 2
]
FILL = [817162, 817061, 816856, 817584]   # four squares completing sum(m^2) = 2^51


def _nearest_bf16_bits(q: Fraction) -> int:
    """bf16 bits of the bf16 value nearest to q > 0 or q < 0 (ties to even),
    by exact rational arithmetic: a second, independent statement of the
    rounding for values in bf16's normal range."""
    sign = 0x8000 if q < 0 else 0
    q = abs(q)
    e = 0
    while q >= 2 * Fraction(2) ** e:
        e += 1
    while q < Fraction(2) ** e:
        e -= 1
    ulp = Fraction(2) ** (e - 7)
    k = q // ulp
    rem = q - k * ulp
    if rem * 2 > ulp or (rem * 2 == ulp and k % 2 == 1):
        k += 1
    v = k * ulp          # the rounded magnitude, 2^e <= v <= 2^(e+1)
    e2 = e + (1 if v == Fraction(2) ** (e + 1) else 0)
    mant = int(v / Fraction(2) ** e2 * 128) - 128
    return sign | ((e2 + 127) << 7) | mant


def _crafted_residual():
    m = [s for s, _ in SPECIAL] + FILL
    rest = 2048 - len(m)
    m += [P if i % 2 == 0 else -P for i in range(rest)]
    bits = [b for _, b in SPECIAL] + [None] * len(FILL) + [0x3F80 if i % 2 == 0 else 0xBF80 for i in range(rest)]
    assert sum(v * v for v in m) == 2 ** 51
    return np.array(m, dtype=np.float32), bits


def test_block_input_rounds_to_bf16_at_midpoints():
    x, bits = _crafted_residual()
    assert np.array_equal(x.astype(np.int64), np.array([int(v) for v in x]))   # exact in fp32
    a = O.block_input(x, FLINT)
    got = (a.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
    assert np.array_equal(a.astype(np.float32).astype(np.float64), a)         # bf16 values are fp32 values
    assert np.all((a.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)     # and have no low bits
    for i, b in enumerate(bits):
        q = Fraction(int(x[i]), P)
        want = _nearest_bf16_bits(q)
        if b is not None:
            assert want == b, (i, hex(want), hex(b))   # the hand-written table agrees with the rule
        assert got[i] == want, (i, int(x[i]), hex(got[i]), hex(want))


def test_block_input_tiny_shape_is_not_rounded():
    """The tiny configuration feeds the normalised fp32 input unrounded."""
    x, _ = _crafted_residual()
    xt = x[:TINY.hidden]
    a = O.block_input(xt, TINY)
    ms = Fraction(sum(int(v) ** 2 for v in xt), TINY.hidden)
    # |a_k| = |x_k| / sqrt(mean(x^2) + 1e-6) to fp64 precision
    rms = float(ms) ** 0.5
    assert np.allclose(a, xt.astype(np.float64) / rms, rtol=1e-15, atol=0)
    assert not np.all((a.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)
