"""GPU parity of the decode attention with learned sinks against the oracle
(TandemLLM "21 Flint", 21.1 table: query heads 32, KV heads 4, head size 128, a
513-position window in a ring of 640 rows on window layers, every position on
full layers; How to Run Flint Locally, "Sinks and the 513-token window").

Seeded synthetic inputs: q, k, v ~ N(0, 1) (k and v stored as bf16), sink
logits U(-9.0, 12.4) in bf16 (the checkpoint's range).

Bound: scores are exact products summed in fp32 inside the matrix cores (the
query in three bf16 parts), so their error is a few fp32 ulps of the sum of
|q_i k_i| / sqrt(128) (about 1e-6 absolute).  The sums of e^(s - m) and of
e^(s - m) v are fp32 in a fixed order over at most 256 positions per chunk (64
for a token that sees at most 768) and
then over the chunks: relative error at most (256 + chunks) 2^-24, 4e-5 at
100,000 positions, typically far less.  1e-4 relative L2 per token still fails
a wrong head group, a dropped sink, a wrong scale or a window off by one
position.
"""
import numpy as np
import pytest
import torch

import flintgen as fg
import int4_expert_ffn_amd as F
from oracle import flint_oracle as O
from parity_util import rel_l2

pytestmark = pytest.mark.gpu
REL_ATT = 1e-4


def bf16_values(bits):
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).double().numpy()


def run_attn(q, kb, vb, sinks, pos, window, ring):
    n = len(pos)
    max_seen = max((p - max(0, p - window + 1) + 1) if window else p + 1 for p in pos)
    wsb = F.flint_attn_workspace_bytes(n, max_seen)
    dev = torch.device("cuda")
    qd = torch.from_numpy(np.ascontiguousarray(q, np.float32)).to(dev)
    kd = torch.from_numpy(np.ascontiguousarray(kb)).to(dev)
    vd = torch.from_numpy(np.ascontiguousarray(vb)).to(dev)
    sd = torch.from_numpy(np.ascontiguousarray(sinks, np.float32)).to(dev)
    out = torch.empty((n, 32, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device=dev)
    F.flint_attn_decode(qd, kd, vd, ring, sd, pos, n, window, out, ws, wsb)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(q, kb, vb, sinks, pos, window, out):
    k, v = bf16_values(kb), bf16_values(vb)
    errs = []
    for t, p in enumerate(pos):
        want = O.attention_decode(q[t].astype(np.float64), k, v, sinks, p, window)
        err = rel_l2(out[t], want)
        assert err <= REL_ATT, (t, p, err)
        errs.append(err)
    return errs


def test_window_layer_positions_and_chunk_edges():
    """Window layer, ring of 640 rows: the first positions (fewer than 513
    visible), the chunk edges 64 / 65 / 256 / 257 / 512 / 513 visible, and
    positions far past the ring's first wrap; all in one call of 12 tokens."""
    ring, W = fg.ATT_RING, fg.ATT_WINDOW
    kb, vb = fg.attn_cache(0, 1, ring)
    sinks = fg.attn_sinks(0, 1)
    pos = [0, 1, 63, 64, 100, 255, 256, 511, 512, 639, 1000, 70000]
    q = fg.attn_queries(0, 1, len(pos))
    out = run_attn(q, kb, vb, sinks, pos, W, ring)
    errs = check(q, kb, vb, sinks, pos, W, out)
    print(f"window layer: rel-L2 max {max(errs):.2e}")


@pytest.mark.parametrize("n_pos", [4096, 100000])
def test_full_layer_long_context(n_pos):
    """Full layer: every position 0 .. pos, the ring as long as the context."""
    kb, vb = fg.attn_cache(0, 2, n_pos)
    sinks = fg.attn_sinks(0, 2)
    pos = [n_pos - 1, n_pos // 2]
    q = fg.attn_queries(0, 2, len(pos))
    out = run_attn(q, kb, vb, sinks, pos, 0, n_pos)
    errs = check(q, kb, vb, sinks, pos, 0, out)
    print(f"full layer, {n_pos} positions: rel-L2 max {max(errs):.2e}")


def test_chunk_size_switch():
    """Tokens seeing at most 768 positions are cut into chunks of 64, longer
    ones into chunks of 256: both sides of the switch (768 / 769 visible) and
    of the chunk edges, in one call and each alone (bitwise)."""
    n_pos = 2048
    kb, vb = fg.attn_cache(0, 6, n_pos)
    sinks = fg.attn_sinks(0, 6)
    pos = [0, 63, 64, 127, 766, 767, 768, 769, 1023, 1024, 2047]
    q = fg.attn_queries(0, 6, len(pos))
    out = run_attn(q, kb, vb, sinks, pos, 0, n_pos)
    for t in range(len(pos)):
        alone = run_attn(q[t:t + 1], kb, vb, sinks, pos[t:t + 1], 0, n_pos)
        assert np.array_equal(alone[0], out[t]), t
    errs = check(q, kb, vb, sinks, pos, 0, out)
    print(f"chunk size switch: rel-L2 max {max(errs):.2e}")


def test_tokens_independent_and_deterministic():
    ring, W = fg.ATT_RING, fg.ATT_WINDOW
    kb, vb = fg.attn_cache(0, 3, ring)
    sinks = fg.attn_sinks(0, 3)
    pos = [700 + 37 * i for i in range(16)]
    q = fg.attn_queries(0, 3, 16)
    all16 = run_attn(q, kb, vb, sinks, pos, W, ring)
    again = run_attn(q, kb, vb, sinks, pos, W, ring)
    assert np.array_equal(all16, again)
    for t in (0, 5, 15):
        alone = run_attn(q[t:t + 1], kb, vb, sinks, pos[t:t + 1], W, ring)
        assert np.array_equal(alone[0], all16[t])


def test_sink_extremes():
    """Sinks at the checkpoint's extremes: at 12.4 the sink takes most of the
    mass (the output shrinks toward 0), at -9 almost none."""
    ring, W = fg.ATT_RING, fg.ATT_WINDOW
    kb, vb = fg.attn_cache(0, 4, ring)
    q = fg.attn_queries(0, 4, 2)
    pos = [3, 900]
    for value in (12.4, -9.0):
        sinks = np.full(32, value, np.float32)
        out = run_attn(q, kb, vb, sinks, pos, W, ring)
        check(q, kb, vb, sinks, pos, W, out)


@pytest.mark.parametrize("n_pos", [20000, 100000])
def test_verify_block_tokens_independent(n_pos):
    """A verify block: tokens at neighbouring positions of a full layer, plus
    one far earlier.  Each token's result must equal the token run alone,
    bitwise, and the oracle."""
    kb, vb = fg.attn_cache(0, 5, n_pos)
    sinks = fg.attn_sinks(0, 5)
    pos = [n_pos - 16 + i for i in range(15)] + [300]
    q = fg.attn_queries(0, 5, len(pos))
    out = run_attn(q, kb, vb, sinks, pos, 0, n_pos)
    for t in (0, 7, 14, 15):
        alone = run_attn(q[t:t + 1], kb, vb, sinks, pos[t:t + 1], 0, n_pos)
        assert np.array_equal(alone[0], out[t]), t
    errs = check(q[[0, 14, 15]], kb, vb, sinks, [pos[0], pos[14], pos[15]], 0, out[[0, 14, 15]])
    print(f"verify block, {n_pos} positions: rel-L2 max {max(errs):.2e}")


def test_writes_stay_inside_workspace_and_out():
    """The call writes nothing past flint_attn_workspace_bytes(n, max_seen) nor
    past out[n]: guard regions after both keep their sentinel, for a window
    call, a mixed call (64- and 256-position chunks) and a long full layer."""
    dev = torch.device("cuda")
    sentinel = 0x7FA5A5A5   # a NaN pattern the kernels never write
    cases = [(fg.ATT_RING, fg.ATT_WINDOW, [5000]), (4096, 0, [100, 700, 769, 4095]), (100000, 0, [99999])]
    for ring, window, pos in cases:
        kb, vb = fg.attn_cache(0, 7, ring)
        sinks = fg.attn_sinks(0, 7)
        q = fg.attn_queries(0, 7, len(pos))
        n = len(pos)
        max_seen = max((p - max(0, p - window + 1) + 1) if window else p + 1 for p in pos)
        wsb = F.flint_attn_workspace_bytes(n, max_seen)
        guard = 4096
        ws = torch.full((wsb // 4 + guard,), sentinel, dtype=torch.int32, device=dev)
        out = torch.full((n * 32 * 128 + guard,), sentinel, dtype=torch.int32, device=dev)
        qd = torch.from_numpy(np.ascontiguousarray(q, np.float32)).to(dev)
        kd = torch.from_numpy(np.ascontiguousarray(kb)).to(dev)
        vd = torch.from_numpy(np.ascontiguousarray(vb)).to(dev)
        sd = torch.from_numpy(np.ascontiguousarray(sinks, np.float32)).to(dev)
        F.flint_attn_decode(qd, kd, vd, ring, sd, pos, n, window, out, ws, wsb)
        torch.cuda.synchronize()
        assert bool((ws[wsb // 4:] == sentinel).all()), (ring, window, pos)
        assert bool((out[n * 32 * 128:] == sentinel).all()), (ring, window, pos)
        res = out[: n * 32 * 128].view(torch.float32).view(n, 32, 128).cpu().numpy()
        check(q, kb, vb, sinks, pos, window, res)
