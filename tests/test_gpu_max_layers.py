"""The largest handle: FLINT_MAX_LAYERS (64) layers, the most any call can run.

Four distinct seeded real-shape layers repeat over the 64 positions (the
library copies each position's weights into its own memory at create, so the
handle really holds 64 layers; repeating the source only saves generation
time).  One token through all 64 layers in one call must equal the chain of
single-layer calls and a split at layer 32 bitwise, and its last layer must
match the oracle teacher-forced; token-group (3 tokens) and prefill (20 tokens)
calls over the 64 layers must match their per-layer chains the same way.
"""
import numpy as np
import pytest
import torch

import flintgen as fg
import int4_expert_ffn_amd as F
from oracle_sources import SynthSource
from parity_util import check_layer, run_forward

pytestmark = pytest.mark.gpu
FL = fg.FLINT
NL = F.FLINT_MAX_LAYERS
NSRC = 4


@pytest.fixture(scope="module")
def deep():
    synth = fg.Synth(FL, seed=11, n_layers=NSRC)
    src_layers = [synth.layer(l, "cuda") for l in range(NSRC)]
    m = F.FlintMoE([src_layers[l % NSRC] for l in range(NL)])
    del src_layers
    torch.cuda.empty_cache()
    ids = torch.full((NL, 20, FL.top_k), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((NL, 20, FL.top_k), dtype=torch.float32, device="cuda")
    m.set_trace(ids, w, 20)
    yield synth, m, ids, w
    m.close()


@pytest.mark.parametrize("n", [1, 3, 20])
def test_all_64_layers_compose_and_last_layer_parity(deep, n):
    synth, m, ids, w = deep
    x0 = fg.tokens(11, range(n))
    full = run_forward(m, x0, 0, NL)
    assert np.all(np.isfinite(full))
    split = run_forward(m, run_forward(m, x0, 0, 32), 32, NL)
    assert np.array_equal(full, split)
    cur = x0
    for l in range(NL - 1):
        cur = run_forward(m, cur, l, l + 1)
    last = run_forward(m, cur, NL - 1, NL)
    assert np.array_equal(full, last)
    # the last layer (source layer (NL - 1) % NSRC) against the oracle
    src = SynthSource(synth)
    for t in range(min(n, 3)):
        check_layer(src, FL, (NL - 1) % NSRC, cur[t], last[t], ids[NL - 1, t].cpu().numpy(),
                    w[NL - 1, t].cpu().numpy(), tight=(n <= 16))
