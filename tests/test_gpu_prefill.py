"""GPU parity of the prefill path (n_tokens > 16: sort by expert, grouped GEMMs
on the matrix cores) against the CPU oracle.

Real Flint shape.  The 2,048-token chunk uses the Zipf-skewed router bias
(b_e = -0.05 * 1.1 * ln r_e), so a few experts get hundreds of tokens and
some very few: the grouped GEMM sees ragged tiles of every size.  Every
token's expert set and weights are checked against the oracle's router; the
block output is checked teacher-forced on a sample of tokens chosen to cover
the heaviest expert, ragged tile tails and the ends of the chunk.
"""
import numpy as np
import pytest
import torch

import flintgen as fg
import int4_expert_ffn_amd as F
from oracle import flint_oracle as O
from oracle_sources import SynthSource
from parity_util import REL_L2_SPEC, check_layer, rel_l2, run_forward, selection_ok

pytestmark = pytest.mark.gpu
FL = fg.FLINT
NMAX = 2048
# Bound for the prefill arithmetic: the decode path's 1e-5 (fp32 accumulation
# of exact products) plus the split of h into two bf16 parts (relative
# truncation <= 2^-17 per element, about 4e-6 on the block output).
REL_L2_PREFILL = 2e-5


def make_model(synth, n_layers):
    m = F.FlintMoE([synth.layer(l, "cuda") for l in range(n_layers)])
    torch.cuda.empty_cache()
    ids = torch.full((n_layers, NMAX, FL.top_k), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((n_layers, NMAX, FL.top_k), dtype=torch.float32, device="cuda")
    m.set_trace(ids, w, NMAX)
    return m, ids, w


@pytest.fixture(scope="module")
def zipf():
    synth = fg.Synth(FL, seed=0, n_layers=2, bias_kind="zipf")
    m, ids, w = make_model(synth, 2)
    yield synth, m, ids, w
    m.close()


@pytest.fixture(scope="module")
def scaled():
    """One layer whose routed up-projection scales are multiplied by 4096 (the
    stack's top layers): SwiGLU outputs pass fp16's range."""
    synth = fg.Synth(FL, seed=7, n_layers=1, up_scale_mult={0: 4096})
    m, ids, w = make_model(synth, 1)
    yield synth, m, ids, w
    m.close()


@pytest.fixture(scope="module")
def uniform():
    synth = fg.Synth(FL, seed=3, n_layers=1)
    m, ids, w = make_model(synth, 1)
    yield synth, m, ids, w
    m.close()


def check_tokens(synth, layer, x, out, ids, w, tokens, bound):
    src = SynthSource(synth)
    errs = []
    for t in tokens:
        err, _ = check_layer(src, FL, layer, x[t], out[t], ids[layer, t].cpu().numpy(), w[layer, t].cpu().numpy(),
                             tight=False)
        errs.append(err)
    assert max(errs) <= bound, (max(errs), bound)
    return errs


@pytest.mark.parametrize("n", [17, 45])
def test_prefill_small_every_token(uniform, n):
    synth, m, ids, w = uniform
    x = fg.tokens(3, range(1000, 1000 + n))
    out = run_forward(m, x, 0, 1)
    errs = check_tokens(synth, 0, x, out, ids, w, range(n), REL_L2_PREFILL)
    print(f"n={n}: rel-L2 max {max(errs):.2e} median {np.median(errs):.2e}")


def test_prefill_2048_zipf(zipf):
    synth, m, ids, w = zipf
    x = fg.tokens(0, range(2000, 2000 + NMAX))
    out = run_forward(m, x, 0, 1)
    assert np.all(np.isfinite(out))
    gids = ids[0, :NMAX].cpu().numpy()
    gw = w[0, :NMAX].cpu().numpy()
    # every token's selection and weights against the oracle's router
    router = synth.router(0).numpy()
    bias = synth.bias(0).numpy()
    near = 0
    for t in range(NMAX):
        r = O.route(O.block_input(x[t], FL), router, bias, FL.top_k)
        assert selection_ok(gids[t], r, FL.top_k), (t, gids[t], r.ids, r.margin)
        if gids[t].tolist() != r.ids.tolist():
            near += 1
            continue
        np.testing.assert_allclose(gw[t], r.weights, rtol=2e-6, atol=0)
    counts = np.bincount(gids.ravel(), minlength=FL.n_experts)
    top = np.sort(counts)[::-1]
    print(f"expert load: top5 {top[:5].tolist()}, median {int(np.median(counts))}, min {counts.min()}, "
          f"empty {int((counts == 0).sum())}; near-tie sets {near}")
    assert counts.sum() == NMAX * FL.top_k
    # block output, teacher-forced, on tokens of the heaviest expert (first and
    # last of its list, i.e. of its first and ragged last tile), of a lightest
    # used expert, and the chunk's ends
    heavy = int(np.argmax(counts))
    light = int(np.flatnonzero(counts == counts[counts > 0].min())[0])
    th = np.flatnonzero((gids == heavy).any(axis=1))
    tl = np.flatnonzero((gids == light).any(axis=1))
    rng = np.random.default_rng(5)
    sample = sorted(set([0, NMAX - 1, int(th[0]), int(th[63]) if len(th) > 63 else int(th[-1]), int(th[-1]),
                         int(tl[0])] + rng.choice(NMAX, 6, replace=False).tolist()))
    errs = check_tokens(synth, 0, x, out, ids, w, sample, REL_L2_PREFILL)
    print(f"sampled tokens {sample}: rel-L2 max {max(errs):.2e}")


def test_prefill_deterministic_in_place_and_composes(zipf):
    synth, m, ids, w = zipf
    x = torch.from_numpy(fg.tokens(0, range(5000, 5300))).cuda()
    a = m.forward(x, 0, 2)
    b = m.forward(x, 0, 2)
    c = x.clone()
    m.forward(c, 0, 2, out=c)
    d = m.forward(m.forward(x, 0, 1), 1, 2)
    torch.cuda.synchronize()
    m.status()
    assert torch.equal(a, b) and torch.equal(a, c) and torch.equal(a, d)


def test_prefill_close_to_decode(uniform):
    """The two paths round differently but compute the same block."""
    synth, m, ids, w = uniform
    x = fg.tokens(3, range(3000, 3017))
    pre = run_forward(m, x, 0, 1)
    for t in range(0, 17, 4):
        dec = run_forward(m, x[t:t + 1], 0, 1)[0]
        assert rel_l2(pre[t] - x[t], dec - x[t]) <= REL_L2_PREFILL


@pytest.mark.parametrize("n", [33, 100, 1000])
def test_prefill_mid_sizes_sampled(uniform, n):
    """Token counts between the small cases and the full chunk: the first, the
    last and a seeded sample of tokens against the oracle."""
    synth, m, ids, w = uniform
    x = fg.tokens(3, range(7000, 7000 + n))
    out = run_forward(m, x, 0, 1)
    assert np.all(np.isfinite(out))
    rng = np.random.default_rng(n)
    sample = sorted(set([0, n - 1] + rng.choice(n, 5, replace=False).tolist()))
    errs = check_tokens(synth, 0, x, out, ids, w, sample, REL_L2_PREFILL)
    print(f"n={n}: sampled rel-L2 max {max(errs):.2e}")


def test_prefill_scaled_up_projection(scaled):
    """x 4096 up-projection scales: h beyond fp16's range, kept as bf16 hi + lo."""
    synth, m, ids, w = scaled
    n = 64
    x = fg.tokens(7, range(n))
    out = run_forward(m, x, 0, 1)
    assert np.all(np.isfinite(out))
    src = SynthSource(synth)
    hmax = 0.0
    for t in (0, 21, 63):
        err, res = check_layer(src, FL, 0, x[t], out[t], ids[0, t].cpu().numpy(), w[0, t].cpu().numpy(),
                               tight=False)
        assert err <= REL_L2_PREFILL, (t, err)
        hmax = max(hmax, res.max_abs_h)
    print(f"max |h| {hmax:.3g}")
    assert hmax > 65504.0


def test_writes_stay_inside_out(uniform):
    """The prefill path writes n_tokens x 2048 floats of out and nothing past
    them (a guard region keeps its sentinel), for a ragged 100-token call and
    the full 2,048-token chunk; the values equal an ordinary call's."""
    synth, m, ids, w = uniform
    sentinel = 0x7FA5A5A5
    for n in (100, NMAX):
        x = torch.from_numpy(fg.tokens(12, range(n))).cuda()
        out = torch.full((n * FL.hidden + 4096,), sentinel, dtype=torch.int32, device="cuda")
        F.flint_moe_forward(m.h, x, n, 0, 1, out, None)
        ref = m.forward(x)
        torch.cuda.synchronize()
        assert bool((out[n * FL.hidden:] == sentinel).all()), n
        assert torch.equal(out[: n * FL.hidden].view(torch.float32).view(n, FL.hidden), ref), n
