"""GPU parity of the output head and of the dense SwiGLU MLP of layers 0 and 1
(int4 matrix-vector products, up to 16 tokens) against the CPU oracle.

Error bounds come from the arithmetic: each code x activation product is exact
in fp32, and a logit (or a gate/up/down row) is an fp32 sum of 2,048 (6,144)
such terms of the form (code + 136) s a, computed as 64 lane sums of 32 terms
then a 6-level tree.  The rounding error is below 3e-6 of the sum of the
terms' magnitudes; the tests allow 1e-5 of it per value, and 1e-5 rel-L2 per
token on the dense MLP's residual update (the decode bound).
"""
import numpy as np
import pytest
import torch

import flintgen as fg
import int4_expert_ffn_amd as F
from oracle import flint_oracle as O

pytestmark = pytest.mark.gpu
FL = fg.FLINT
H = FL.hidden
REL_L2 = 1e-5


def magnitude_bound(codes, scales, a):
    """sum_k |(code + 136) s a_k| per row: the scale of the fp32 rounding error."""
    v = O.unpack_int4(codes).astype(np.float64) + 136.0
    s = np.repeat(O.bf16_bits_to_f64(scales), FL.group, axis=-1)
    return np.abs(v * s) @ np.abs(a)


# ------------------------------------------------------------------ head
@pytest.fixture(scope="module")
def head():
    c, s = fg.head(0, device="cuda")
    torch.cuda.synchronize()
    return c, s


def run_head(c, s, rows, x_np):
    x = torch.from_numpy(np.ascontiguousarray(x_np, np.float32)).cuda()
    out = torch.full((x.shape[0], rows), float("nan"), dtype=torch.float32, device="cuda")
    F.flint_head_forward(F.q4(c, s), rows, x, x.shape[0], out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_head_rows(x_np, logits, rows_idx, codes, scales):
    for t in range(x_np.shape[0]):
        ref = O.head_logits(x_np[t], codes, scales, FL)
        bound = 1e-5 * magnitude_bound(codes, scales, O.block_input(x_np[t], FL))
        err = np.abs(logits[t, rows_idx].astype(np.float64) - ref)
        assert np.all(err <= bound), (t, float(np.max(err / bound)))


def test_head_full_vocabulary_sampled_rows(head):
    c, s = head
    rng = np.random.default_rng(0)
    idx = np.unique(np.concatenate([np.arange(8), fg.VOCAB - 8 + np.arange(8), rng.choice(fg.VOCAB, 48, replace=False)]))
    cc, ss = fg.head(0, row_ids=idx.tolist())
    x = fg.tokens(0, range(40, 44))
    out = run_head(c, s, fg.VOCAB, x)
    assert np.all(np.isfinite(out))
    check_head_rows(x, out, idx, cc.numpy(), ss.numpy())


@pytest.mark.parametrize("rows", [1, 3, 1000, 4097])
def test_head_ragged_row_counts_every_row(head, rows):
    c, s = head
    cc, ss = fg.head(0, rows=rows)
    x = fg.tokens(1, range(3))
    out = run_head(c, s, rows, x)
    check_head_rows(x, out, np.arange(rows), cc.numpy(), ss.numpy())


def test_head_batch_invariance_and_zero_input(head):
    c, s = head
    x = fg.tokens(2, range(16))
    singles = np.stack([run_head(c, s, fg.VOCAB, x[t:t + 1])[0] for t in (0, 5, 15)])
    full = run_head(c, s, fg.VOCAB, x)
    assert np.array_equal(full[[0, 5, 15]], singles)
    assert np.array_equal(run_head(c, s, fg.VOCAB, x[:4])[[0]], singles[[0]])
    z = run_head(c, s, 4097, np.zeros((2, H), np.float32))
    assert np.all(z == 0)


# ------------------------------------------------------------------ dense MLP
@pytest.fixture(scope="module", params=[fg.DENSE_MLP_SIZE, 2048])
def dense(request):
    inter = request.param
    w = fg.dense_layer(0, 1, device="cuda", inter=inter)
    torch.cuda.synchronize()
    wc = {k: v.cpu().numpy() for k, v in w.items()}
    return inter, w, wc


def run_dense(inter, w, x_np, out_is_x=False):
    x = torch.from_numpy(np.ascontiguousarray(x_np, np.float32)).cuda()
    n = x.shape[0]
    h = torch.full((n, inter), float("nan"), dtype=torch.float32, device="cuda")
    out = x if out_is_x else torch.full_like(x, float("nan"))
    F.flint_dense_mlp_forward(F.q4(w["gate"], w["gate_s"]), F.q4(w["up"], w["up_s"]), F.q4(w["down"], w["down_s"]),
                              inter, x, n, h, out)
    torch.cuda.synchronize()
    return h.cpu().numpy(), out.cpu().numpy()


def test_dense_mlp_parity(dense):
    inter, w, wc = dense
    x = fg.tokens(3, range(5))
    h, out = run_dense(inter, w, x)
    for t in range(len(x)):
        res = O.dense_mlp(x[t], wc, FL)
        a = O.block_input(x[t], FL)
        # h: silu(g) u from two rows with the bound above (silu is 1-Lipschitz-ish: |silu'| <= 1.1)
        bg = magnitude_bound(wc["gate"], wc["gate_s"], a)
        bu = magnitude_bound(wc["up"], wc["up_s"], a)
        g = O.dequant(wc["gate"], wc["gate_s"], FL.group) @ a
        u = O.dequant(wc["up"], wc["up_s"], FL.group) @ a
        hb = 1e-5 * (1.1 * bg * np.abs(u) + np.abs(O.silu(g)) * bu) + 1e-6 * np.abs(res.h)
        assert np.all(np.abs(h[t] - res.h) <= hb), (t, float(np.max(np.abs(h[t] - res.h) / hb)))
        d_gpu = out[t].astype(np.float64) - x[t]
        d_ref = res.x_out.astype(np.float64) - x[t]
        err = np.linalg.norm(d_gpu - d_ref) / np.linalg.norm(d_ref)
        assert err <= REL_L2, (t, err)
    print(f"inter={inter}: max |h| {np.abs(h).max():.3g}")


def test_dense_mlp_batch_invariance_in_place_and_zero(dense):
    """Every token's h and out are bitwise the same for any token count (1, 2,
    3, 4, 7 and 16 tokens per call), also in place (out = x)."""
    inter, w, wc = dense
    x = fg.tokens(4, range(16))
    h1, o1 = run_dense(inter, w, x[:1])
    h4, o4 = run_dense(inter, w, x[:4])
    h7, o7 = run_dense(inter, w, x[:7])
    h16, o16 = run_dense(inter, w, x)
    assert np.array_equal(h16[:1], h1) and np.array_equal(o16[:1], o1)
    assert np.array_equal(h16[:4], h4) and np.array_equal(o16[:4], o4)
    assert np.array_equal(h16[:7], h7) and np.array_equal(o16[:7], o7)
    hi, oi = run_dense(inter, w, x, out_is_x=True)
    assert np.array_equal(hi, h16) and np.array_equal(oi, o16)
    hi3, oi3 = run_dense(inter, w, x[:3], out_is_x=True)
    assert np.array_equal(hi3, h16[:3]) and np.array_equal(oi3, o16[:3])
    hz, oz = run_dense(inter, w, np.zeros((3, H), np.float32))
    assert np.all(hz == 0) and np.all(oz == 0)
    h2, o2 = run_dense(inter, w, x[4:6])
    assert np.array_equal(h2, h16[4:6]) and np.array_equal(o2, o16[4:6])


def test_dense_mlp_power_of_two_up_scale_is_exact(dense):
    inter, w, wc = dense
    x = fg.tokens(5, range(2))
    h, _ = run_dense(inter, w, x)
    w2 = dict(w, up_s=(w["up_s"].to(torch.int32) + (3 << 7)).to(torch.int16))
    h2, _ = run_dense(inter, w2, x)
    assert np.array_equal(h2, h * 8.0)


def test_writes_stay_inside_outputs(head, dense):
    """The head writes n x rows logits and the dense MLP n x inter of h and
    n x 2048 of out, nothing past them (guard regions keep their sentinel),
    with a ragged row count for the head."""
    sentinel = 0x7FA5A5A5
    c, s = head
    x = torch.from_numpy(fg.tokens(13, range(3))).cuda()
    rows = 1000
    logits = torch.full((3 * rows + 4096,), sentinel, dtype=torch.int32, device="cuda")
    F.flint_head_forward(F.q4(c, s), rows, x, 3, logits)
    torch.cuda.synchronize()
    assert bool((logits[3 * rows:] == sentinel).all())
    inter, w, wc = dense
    h = torch.full((3 * inter + 4096,), sentinel, dtype=torch.int32, device="cuda")
    out = torch.full((3 * H + 4096,), sentinel, dtype=torch.int32, device="cuda")
    F.flint_dense_mlp_forward(F.q4(w["gate"], w["gate_s"]), F.q4(w["up"], w["up_s"]), F.q4(w["down"], w["down_s"]),
                              inter, x, 3, h, out)
    torch.cuda.synchronize()
    assert bool((h[3 * inter:] == sentinel).all())
    assert bool((out[3 * H:] == sentinel).all())
    h_ref, out_ref = run_dense(inter, w, x.cpu().numpy())
    assert np.array_equal(h[: 3 * inter].view(torch.float32).view(3, inter).cpu().numpy(), h_ref)
    assert np.array_equal(out[: 3 * H].view(torch.float32).view(3, H).cpu().numpy(), out_ref)


def _pack_rows(codes):
    """int4 codes [rows][K] in [-8, 7] -> bytes [rows][K/2], even k in the low nibble."""
    c = (np.asarray(codes, np.int64) & 0xF).astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def test_dense_mlp_block_input_at_bf16_midpoints():
    """A residual whose normalised values are exact and land on (and next to)
    bf16 rounding midpoints, so the block input takes its exact-quotient path.
    Gate and up rows r < 16 pick element r alone (code 1, scale 1), so h_r =
    silu(a_r) a_r shows a_r itself: one bf16 step in a_r (2^-8 relative)
    moves h_r by far more than the bound used here."""
    from test_oracle_stack_pins import _crafted_residual
    x, _ = _crafted_residual()
    inter = 2048
    gu = np.zeros((inter, H), np.int64)
    gu[np.arange(16), np.arange(16)] = 1
    one = np.full((inter, H // FL.group), 0x3F80, np.int16)   # scale 1.0
    dn = fg.dense_layer(0, 1, inter=inter)
    wc = {"gate": _pack_rows(gu), "gate_s": one, "up": _pack_rows(gu), "up_s": one,
          "down": dn["down"].numpy(), "down_s": dn["down_s"].numpy()}
    w = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in wc.items()}
    xs = np.stack([x, fg.token(6, 0)])   # a second, ordinary token in the same call
    h, out = run_dense(inter, w, xs)
    res = O.dense_mlp(x, wc, FL)
    a = O.block_input(x, FL)
    assert np.all(np.abs(h[0, :16] - res.h[:16]) <= 2e-4), np.abs(h[0, :16] - res.h[:16]).max()
    # a one-step error in any of the first 16 activations would exceed the bound above
    step = np.abs(a[:16]) * 2.0 ** -8
    assert np.all(step * 0.9 > 2e-4 * 2)
    d_gpu = out[0].astype(np.float64) - x
    d_ref = res.x_out.astype(np.float64) - x
    assert np.linalg.norm(d_gpu - d_ref) / np.linalg.norm(d_ref) <= REL_L2
    h1, _ = run_dense(inter, w, xs[1:])
    assert np.array_equal(h1[0], h[1])
