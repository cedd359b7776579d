"""GPU parity of the fp16-intermediate form (TandemLLM "21 Flint", 21.2: packs
divide each routed expert's up projection by expert_interm_div = 128 so SwiGLU
outputs fit fp16, and the routing weights carry the factor back) against the
oracle's form, and its distance from the fp32 path.

Real Flint shape, seeded synthetic weights: the pack form is the same weights
with every routed up-projection scale divided by 128 (exact in bf16).
"""
import numpy as np
import pytest
import torch

import flintgen as fg
import int4_expert_ffn_amd as F
from oracle import flint_oracle as O
from oracle_sources import SynthSource
from parity_util import build_layers, rel_l2, run_forward, selection_ok

pytestmark = pytest.mark.gpu
FL = fg.FLINT
DIV = 128
N_LAYERS = 3
# GPU and oracle round the same SwiGLU outputs to fp16, from fp32 and fp64
# values about 1e-7 apart (relative): a value that close to a rounding boundary
# lands one fp16 ulp (2^-10 relative) away, about 4e-4 of the 4,096 values of a
# token-layer, i.e. a couple; each moves the output by 2^-10 of one of 4,096
# terms, so rel-L2 ~ 2^-10 sqrt(2 / 4096) ~ 2e-5, plus the fp32 path's 1e-6.
# 1e-4 leaves a 5x margin and still fails a missed rounding (2.4e-4) or a
# dropped divisor.
REL_L2_FP16H = 1e-4


@pytest.fixture(scope="module")
def models():
    pack = fg.Synth(FL, seed=0, n_layers=N_LAYERS, up_scale_div=DIV)
    std = fg.Synth(FL, seed=0, n_layers=N_LAYERS)
    layers = build_layers(pack, range(N_LAYERS))
    m16 = F.FlintMoE(layers, interm_div=DIV)
    del layers
    layers = build_layers(std, range(N_LAYERS))
    m32 = F.FlintMoE(layers)
    del layers
    torch.cuda.empty_cache()
    ids = torch.full((N_LAYERS, 16, 6), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((N_LAYERS, 16, 6), dtype=torch.float32, device="cuda")
    m16.set_trace(ids, w, 16)
    yield pack, m16, m32, ids, w
    m16.close()
    m32.close()


def check_layer_fp16(src, layer, x_in, x_out, gpu_ids, gpu_w):
    a = O.block_input(x_in, FL)
    res = O.moe_block_fp16_interm(a, src, layer, FL, DIV)
    gpu_ids = [int(e) for e in gpu_ids]
    assert selection_ok(gpu_ids, res.route, FL.top_k), (layer, gpu_ids, res.route.ids)
    if gpu_ids != res.route.ids.tolist():
        res = O.moe_block_fp16_interm(a, src, layer, FL, DIV, forced=gpu_ids)
    np.testing.assert_allclose(gpu_w, res.route.weights, rtol=2e-6, atol=0)   # traced weights are unscaled
    x_ref = (x_in.astype(np.float64) + res.delta).astype(np.float32)
    err = rel_l2(x_out.astype(np.float64) - x_in, x_ref.astype(np.float64) - x_in)
    assert err <= REL_L2_FP16H, (layer, err)
    return err, res


def test_fp16_interm_layer_parity(models):
    pack, m16, m32, ids, w = models
    src = SynthSource(pack)
    errs = []
    for t in range(4):
        cur = fg.token(0, 900 + t)[None]
        for l in range(N_LAYERS):
            nxt = run_forward(m16, cur, l, l + 1)
            err, _ = check_layer_fp16(src, l, cur[0], nxt[0], ids[l, 0].cpu().numpy(), w[l, 0].cpu().numpy())
            errs.append(err)
            cur = nxt
    print(f"fp16 form vs oracle: rel-L2 max {max(errs):.2e}, median {np.median(errs):.2e}")


def test_fp16_interm_vs_fp32_path(models):
    """The numerics cost of fp16 intermediates: both forms on the same layer
    input (the fp32 path's residual, so both route alike).  Round-to-nearest
    errors have an rms of at most 2^-11 / sqrt(3) of |h| (about 2.8e-4 of the
    block output); 6e-4 allows twice that.  End to end over the three layers
    is printed, not bounded: the forms may pick different experts at a near
    tie."""
    pack, m16, m32, ids, w = models
    rels, e2e = [], []
    for t in range(8):
        x0 = fg.token(0, 950 + t)[None]
        cur = x0
        for l in range(N_LAYERS):
            a = run_forward(m16, cur, l, l + 1)
            b = run_forward(m32, cur, l, l + 1)
            rels.append(rel_l2(a[0].astype(np.float64) - cur[0], b[0].astype(np.float64) - cur[0]))
            cur = b
        a = run_forward(m16, x0, 0, N_LAYERS)
        e2e.append(rel_l2(a[0].astype(np.float64) - x0[0], cur[0].astype(np.float64) - x0[0]))
    print(f"fp16 vs fp32 intermediates per layer: rel-L2 max {max(rels):.2e}, median {np.median(rels):.2e}; "
          f"3 layers end to end: max {max(e2e):.2e}, median {np.median(e2e):.2e}")
    assert max(rels) <= 6e-4
    assert min(rels) > 1e-6      # the rounding is there


def test_fp16_interm_scaled_layer_needs_the_divisor():
    """A layer with x4096 routed up scales: SwiGLU outputs pass fp16's range.
    The pack form (/128) stays finite and matches the oracle; the same fp16
    form on undivided weights overflows."""
    raw = fg.Synth(FL, seed=7, n_layers=1, up_scale_mult={0: 4096})
    pack = fg.Synth(FL, seed=7, n_layers=1, up_scale_mult={0: 4096}, up_scale_div=DIV)
    x = fg.tokens(7, range(3))
    m = F.FlintMoE(build_layers(pack, [0]), interm_div=DIV)
    try:
        ids = torch.full((1, 1, 6), -1, dtype=torch.int32, device="cuda")
        w = torch.zeros((1, 1, 6), dtype=torch.float32, device="cuda")
        m.set_trace(ids, w, 1)
        src = SynthSource(pack)
        hmax = 0.0
        for t in range(3):
            out = run_forward(m, x[t:t + 1], 0, 1)
            assert np.all(np.isfinite(out))
            _, res = check_layer_fp16(src, 0, x[t], out[0], ids[0, 0].cpu().numpy(), w[0, 0].cpu().numpy())
            hmax = max(hmax, res.max_abs_h)
        print(f"max |h| in fp16 after /{DIV}: {hmax:.3g}")
    finally:
        m.close()
    m = F.FlintMoE(build_layers(raw, [0]), interm_div=1)
    try:
        out = run_forward(m, x[:1], 0, 1)
        assert not np.all(np.isfinite(out))
    finally:
        m.close()


def test_fp16_interm_deterministic_and_decode_only(models):
    """Deterministic; implemented for calls of up to 16 tokens (the prefill
    path above that returns FLINT_ERR_UNSUPPORTED)."""
    pack, m16, m32, ids, w = models
    x = torch.from_numpy(fg.tokens(0, [990])).cuda()
    a = m16.forward(x)
    b = m16.forward(x)
    torch.cuda.synchronize()
    m16.status()
    assert torch.equal(a, b)
    with pytest.raises(F.FlintMoEError) as ei:
        m16.forward(torch.zeros((17, FL.hidden), device="cuda"))
    assert ei.value.code == F.FLINT_ERR_UNSUPPORTED


@pytest.mark.parametrize("n", [2, 3, 5, 6, 8, 9, 10, 12, 16])
def test_fp16_interm_token_groups_match_single_tokens(models, n):
    """Several tokens per call (every group kernel: 2, 4 and 8 and 16 tokens
    per group size, exact ranges for 5, 6, 9, 10 and 12, each with its own
    batch count): each token's output over the three layers is bitwise the
    one-token call's."""
    pack, m16, m32, ids, w = models
    x = torch.from_numpy(fg.tokens(2, range(100, 100 + n))).cuda()
    together = m16.forward(x)
    for t in sorted({0, n // 2, n - 1}):
        alone = m16.forward(x[t:t + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(alone[0], together[t]), (n, t)


def test_fp16_interm_token_group_layer_parity(models):
    """A four-token call against the oracle's form, teacher-forced per layer
    and token."""
    pack, m16, m32, ids, w = models
    src = SynthSource(pack)
    cur = fg.tokens(2, range(200, 204))
    errs = []
    for l in range(N_LAYERS):
        nxt = run_forward(m16, cur, l, l + 1)
        for t in range(4):
            err, _ = check_layer_fp16(src, l, cur[t], nxt[t], ids[l, t].cpu().numpy(), w[l, t].cpu().numpy())
            errs.append(err)
        cur = nxt
    print(f"fp16 form, 4-token calls vs oracle: rel-L2 max {max(errs):.2e}")
