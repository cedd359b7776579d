"""The allocation-free decode attention (flint_attn_decode_noalloc, for callers
that cannot allocate device memory around the call) against the workspace
entry point it mirrors: bitwise equal outputs on two calls in a row, the
second smaller than the first (the scratch array keeps the first call's
partials, which the second must not read), and the size limit enforced.
"""
import numpy as np
import pytest
import torch

import flintgen as fg
import int4_expert_ffn_amd as F

pytestmark = pytest.mark.gpu


def _inputs(ring, layer, n):
    dev = torch.device("cuda")
    kb, vb = fg.attn_cache(0, layer, ring)
    sinks = fg.attn_sinks(0, layer)
    q = fg.attn_queries(0, layer, n)
    to = lambda a, dt=None: torch.from_numpy(np.ascontiguousarray(a if dt is None else a.astype(dt))).to(dev)
    return to(q, np.float32), to(kb), to(vb), to(sinks, np.float32)


def _with_workspace(q, k, v, ring, s, pos, window):
    n = len(pos)
    max_seen = max((p - max(0, p - window + 1) + 1) if window else p + 1 for p in pos)
    wsb = F.flint_attn_workspace_bytes(n, max_seen)
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device="cuda")
    out = torch.empty((n, 32, 128), dtype=torch.float32, device="cuda")
    F.flint_attn_decode(q, k, v, ring, s, pos, n, window, out, ws, wsb)
    return out


def _no_alloc(q, k, v, ring, s, pos, window):
    out = torch.empty((len(pos), 32, 128), dtype=torch.float32, device="cuda")
    F.flint_attn_decode_noalloc(q, k, v, ring, s, pos, len(pos), window, out)
    return out


def test_no_alloc_matches_workspace_entry_point_on_consecutive_calls():
    # first call: 16 tokens of a full layer (many chunks each), then a
    # smaller call: 3 tokens, fewer chunks
    ring = 12000
    q, k, v, s = _inputs(ring, 3, 16)
    pos_a = [11999 - 700 * i for i in range(16)]
    pos_b = [5000, 300, 769]
    a = _no_alloc(q, k, v, ring, s, pos_a, 0)
    b = _no_alloc(q[:3], k, v, ring, s, pos_b, 0)
    ra = _with_workspace(q, k, v, ring, s, pos_a, 0)
    rb = _with_workspace(q[:3], k, v, ring, s, pos_b, 0)
    torch.cuda.synchronize()
    assert torch.equal(a, ra)
    assert torch.equal(b, rb)
    # a window layer after them, one token
    wq, wk, wv, ws = _inputs(fg.ATT_RING, 4, 1)
    c = _no_alloc(wq, wk, wv, fg.ATT_RING, ws, [90000], fg.ATT_WINDOW)
    rc = _with_workspace(wq, wk, wv, fg.ATT_RING, ws, [90000], fg.ATT_WINDOW)
    torch.cuda.synchronize()
    assert torch.equal(c, rc)


def test_no_alloc_rejects_calls_beyond_its_scratch():
    ring = 16000
    q, k, v, s = _inputs(ring, 5, 16)
    out = torch.empty((16, 32, 128), dtype=torch.float32, device="cuda")
    # 16 tokens seeing 15,873 positions each need more than the 16 MiB it holds
    with pytest.raises(F.FlintMoEError) as ei:
        F.flint_attn_decode_noalloc(q, k, v, ring, s, [15872] * 16, 16, 0, out)
    assert ei.value.code == F.FLINT_ERR_INVALID_ARG
    assert F.flint_attn_workspace_bytes(16, 15873) > F.FLINT_ATT_SCRATCH_BYTES
    # the largest size it takes still runs and matches
    a = _no_alloc(q, k, v, ring, s, [15871] * 16, 0)
    ra = _with_workspace(q, k, v, ring, s, [15871] * 16, 0)
    torch.cuda.synchronize()
    assert torch.equal(a, ra)
