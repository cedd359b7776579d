"""GPU parity of the decode path (n_tokens <= 16) against the CPU oracle.

Real Flint shape (hidden 2048, 256 experts of 512, top-6, shared 1024, int4
group 128), seeded synthetic weights, three layers.  Each layer is checked
teacher-forced: the oracle takes the GPU's input residual of that layer.
"""
import os

import numpy as np
import pytest
import torch

import flintgen as fg
import int4_expert_ffn_amd as F
from oracle_sources import SynthSource
from parity_util import build_layers, run_forward
from parity_util import check_layer as _check_layer

pytestmark = pytest.mark.gpu
FL = fg.FLINT
N_LAYERS = 3
CAP = 16


@pytest.fixture(scope="module")
def model():
    synth = fg.Synth(FL, seed=0, n_layers=N_LAYERS)
    layers = build_layers(synth, range(N_LAYERS))
    m = F.FlintMoE(layers)
    del layers
    torch.cuda.empty_cache()
    ids = torch.full((N_LAYERS, CAP, 6), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((N_LAYERS, CAP, 6), dtype=torch.float32, device="cuda")
    m.set_trace(ids, w, CAP)
    yield synth, m, ids, w
    m.close()


def run(m, x_np, l0, l1):
    return run_forward(m, x_np, l0, l1)


def check_layer(synth, layer, x_in, x_out, gpu_ids, gpu_w, tight=True):
    return _check_layer(SynthSource(synth), FL, layer, x_in, x_out, gpu_ids, gpu_w, tight)


def test_one_layer_parity(model):
    synth, m, ids, w = model
    errs = []
    for t in range(6):
        x = fg.token(0, t)[None]
        out = run(m, x, 0, 1)
        err, _ = check_layer(synth, 0, x[0], out[0], ids[0, 0].cpu().numpy(), w[0, 0].cpu().numpy())
        errs.append(err)
    print("rel-L2 per token:", ["%.2e" % e for e in errs])


def test_stack_composes_and_matches_per_layer(model):
    synth, m, ids, w = model
    x = fg.tokens(0, [100, 101])
    full = run(m, x, 0, N_LAYERS)
    tr_ids, tr_w = ids.cpu().numpy().copy(), w.cpu().numpy().copy()
    cur = x
    for l in range(N_LAYERS):
        nxt = run(m, cur, l, l + 1)
        for t in range(2):
            assert np.array_equal(ids[l, t].cpu().numpy(), tr_ids[l, t])
            check_layer(synth, l, cur[t], nxt[t], tr_ids[l, t], tr_w[l, t])
        cur = nxt
    assert np.array_equal(cur, full)     # layer ranges compose bitwise


def test_batch_invariance_bitwise(model):
    synth, m, ids, w = model
    x = fg.tokens(0, range(200, 200 + CAP))
    singles, sids = [], []
    for t in range(CAP):
        singles.append(run(m, x[t:t + 1], 0, N_LAYERS)[0])
        sids.append(ids[:, 0].cpu().numpy().copy())
    # every decode kernel variant: one token; token groups of 2, 4, 8, 16 with
    # and without idle groups (3, 7, 13); exact workgroup ranges with each
    # batch count the host picks (5: 3 pairs, 6: 4, 9: 5, 10: 6, 12: 7)
    for n in (2, 3, 4, 5, 6, 7, 9, 10, 12, 13, CAP):
        out = run(m, x[:n], 0, N_LAYERS)
        for t in range(n):
            assert np.array_equal(out[t], singles[t]), (n, t)
            assert np.array_equal(ids[:, t].cpu().numpy(), sids[t]), (n, t)


def test_largest_decode_batch_parity(model):
    """16 tokens in one call (the largest decode batch, up to 96 distinct
    experts per layer): every token of every layer against the oracle."""
    synth, m, ids, w = model
    x = fg.tokens(0, range(600, 600 + CAP))
    cur = x
    for l in range(N_LAYERS):
        nxt = run(m, cur, l, l + 1)
        for t in range(CAP):
            check_layer(synth, l, cur[t], nxt[t], ids[l, t].cpu().numpy(), w[l, t].cpu().numpy())
        cur = nxt
    distinct = len(set(ids[0].cpu().numpy().ravel().tolist()))
    print(f"distinct experts in layer 0: {distinct}")


def test_determinism_and_in_place(model):
    synth, m, ids, w = model
    x = torch.from_numpy(fg.tokens(0, range(300, 305))).cuda()
    a = m.forward(x, 0, N_LAYERS)
    b = m.forward(x, 0, N_LAYERS)
    c = x.clone()
    m.forward(c, 0, N_LAYERS, out=c)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


def test_zero_input(model):
    synth, m, ids, w = model
    out = run(m, np.zeros((2, FL.hidden), np.float32), 0, N_LAYERS)
    assert np.all(out == 0)
    for l in range(N_LAYERS):
        b = synth.bias(l).numpy().astype(np.float64)
        want = sorted(range(FL.n_experts), key=lambda e: (-b[e], e))[:FL.top_k]
        assert ids[l, 0].cpu().numpy().tolist() == want


def test_invalid_arguments_rejected(model):
    synth, m, ids, w = model
    x = torch.zeros((4, FL.hidden), device="cuda")
    out = torch.zeros_like(x)
    bad = [
        (x, 0, 0, 1, out), (x, 2049, 0, 1, out), (x, 1, -1, 1, out), (x, 1, 1, 1, out),
        (x, 1, 0, N_LAYERS + 1, out),
    ]
    for args in bad:
        with pytest.raises(F.FlintMoEError) as ei:
            F.flint_moe_forward(m.h, args[0], args[1], args[2], args[3], args[4])
        assert ei.value.code == F.FLINT_ERR_INVALID_ARG
    with pytest.raises(F.FlintMoEError) as ei:     # misaligned
        F.flint_moe_forward(m.h, x.data_ptr() + 4, 1, 0, 1, out)
    assert ei.value.code == F.FLINT_ERR_INVALID_ARG
    with pytest.raises(F.FlintMoEError) as ei:     # partial overlap
        F.flint_moe_forward(m.h, x, 2, 0, 1, x.data_ptr() + 4 * FL.hidden)
    assert ei.value.code == F.FLINT_ERR_INVALID_ARG
    with pytest.raises(F.FlintMoEError) as ei:     # above the trace capacity
        F.flint_moe_forward(m.h, torch.zeros((CAP + 1, FL.hidden), device="cuda"), CAP + 1, 0, 1,
                            torch.zeros((CAP + 1, FL.hidden), device="cuda"))
    assert ei.value.code == F.FLINT_ERR_INVALID_ARG
    torch.cuda.synchronize()
    m.status()


CREATE_ALLOCATIONS = 10   # device allocations of one create call
RUNTIME_CHUNKS = 2 * (2 << 20)   # two of the HIP runtime's 2 MiB small-buffer chunks


def test_allocation_failure_is_reported_and_releases_everything(model):
    """Create failing at each of its device allocations in turn: the error is
    reported, and what the call had allocated until then is freed.  The
    library's own count of live device allocations is exact; device-level free
    memory is checked one-sided only, since the HIP runtime may keep freed
    blocks for reuse and return them to the device later (a block freed by an
    earlier destroy has come back during a later create), and keeps the 2 MiB
    chunks it carves small buffers from, so free memory can rise between the
    steps but must never fall below where it started by more than two such
    chunks."""
    synth, m, ids, w = model
    layers = build_layers(fg.Synth(FL, seed=1, n_layers=1), [0])
    x = torch.from_numpy(fg.tokens(0, [7])).cuda()

    def create_run_close():
        m2 = F.FlintMoE(layers)
        assert F.flint_moe_debug_live_allocations() == live0 + CREATE_ALLOCATIONS
        out = m2.forward(x, 0, 1)
        torch.cuda.synchronize()
        m2.status()
        m2.close()
        return out

    live0 = F.flint_moe_debug_live_allocations()   # the module's model holds its own
    create_run_close()   # first: the runtime's lazy set-up (e.g. of the first cooperative launch) is done
    assert F.flint_moe_debug_live_allocations() == live0
    torch.cuda.empty_cache()
    free0 = torch.cuda.mem_get_info()[0]
    try:
        for k in range(1, CREATE_ALLOCATIONS + 1):
            os.environ["FLINT_MOE_FAIL_ALLOC"] = str(k)
            with pytest.raises(F.FlintMoEError) as ei:
                F.FlintMoE(layers)
            assert ei.value.code == F.FLINT_ERR_OUT_OF_MEMORY
            assert f"allocation {k} " in str(ei.value)
            assert F.flint_moe_debug_live_allocations() == live0, k
            assert torch.cuda.mem_get_info()[0] >= free0 - RUNTIME_CHUNKS, k
        os.environ["FLINT_MOE_FAIL_ALLOC"] = str(CREATE_ALLOCATIONS + 1)   # past the last one: no failure
        out = create_run_close()
    finally:
        del os.environ["FLINT_MOE_FAIL_ALLOC"]
    assert torch.isfinite(out).all()
    assert F.flint_moe_debug_live_allocations() == live0
    del out
    torch.cuda.empty_cache()            # the output tensor was torch's, not the library's
    # the runtime carves the small buffers (error word, layer table) from 2 MiB
    # chunks that it keeps once made; the exact check is the count above
    assert torch.cuda.mem_get_info()[0] >= free0 - RUNTIME_CHUNKS


def test_persistent_and_layered_modes_agree_bitwise(model):
    """The persistent kernel (one launch per call, tagged exchanges between
    workgroups) and the per-layer kernels run the same arithmetic."""
    synth, m, ids, w = model
    layers = build_layers(synth, range(N_LAYERS))
    os.environ["FLINT_MOE_DECODE"] = "layered"
    try:
        m2 = F.FlintMoE(layers)
    finally:
        del os.environ["FLINT_MOE_DECODE"]
    del layers
    x = torch.from_numpy(fg.tokens(0, range(400, 416))).cuda()
    try:
        for n in (1, 4, 9, 16):
            a = m.forward(x[:n])
            b = m2.forward(x[:n])
            torch.cuda.synchronize()
            assert torch.equal(a, b), n
        m.status()
        m2.status()
    finally:
        m2.close()


def test_single_token_exchange_slots_across_mixed_calls(model):
    """Single-token calls pass x and h between workgroups through per-layer
    slots of two call parities, each call re-arming the other parity's slots.
    A queued mix of single-token calls over varied layer ranges, with token
    group calls between them, must match the per-layer kernels bitwise; a slot
    left holding an earlier call's value would be read as fresh and show here."""
    synth, m, ids, w = model
    layers = build_layers(synth, range(N_LAYERS))
    os.environ["FLINT_MOE_DECODE"] = "layered"
    try:
        ref = F.FlintMoE(layers)
    finally:
        del os.environ["FLINT_MOE_DECODE"]
    del layers
    rng = np.random.default_rng(11)
    x = torch.from_numpy(fg.tokens(0, range(700, 716))).cuda()
    calls = []
    for i in range(30):
        n = int(rng.choice([1, 1, 1, 2, 5]))
        l0 = int(rng.integers(0, N_LAYERS))
        l1 = int(rng.integers(l0 + 1, N_LAYERS + 1))
        t0 = int(rng.integers(0, 16 - n + 1))
        calls.append((n, l0, l1, t0))
    try:
        outs = [m.forward(x[t0:t0 + n], l0, l1) for n, l0, l1, t0 in calls]   # queued, no sync between
        refs = [ref.forward(x[t0:t0 + n], l0, l1) for n, l0, l1, t0 in calls]
        torch.cuda.synchronize()
        m.status()
        ref.status()
        for i, (a, b) in enumerate(zip(outs, refs)):
            assert torch.equal(a, b), (i, calls[i])
    finally:
        ref.close()


def test_writes_stay_inside_out(model):
    """flint_moe_forward writes n_tokens x 2048 floats of out and nothing past
    them (a guard region keeps its sentinel): the one-token kernel, a token-group
    call and the largest decode batch; the values equal an ordinary call's."""
    synth, m, ids, w = model
    sentinel = 0x7FA5A5A5   # a NaN pattern the kernels never write
    for n in (1, 5, CAP):
        x = torch.from_numpy(fg.tokens(11, range(n))).cuda()
        out = torch.full((n * FL.hidden + 4096,), sentinel, dtype=torch.int32, device="cuda")
        F.flint_moe_forward(m.h, x, n, 0, N_LAYERS, out, None)
        ref = m.forward(x)
        torch.cuda.synchronize()
        assert bool((out[n * FL.hidden:] == sentinel).all()), n
        assert torch.equal(out[: n * FL.hidden].view(torch.float32).view(n, FL.hidden), ref), n


def test_exchange_tag_wrap_clears_buffers_and_keeps_results(model):
    """Decode calls tag exchanged words with a per-call counter; where it would
    wrap, the call clears the exchange buffers and restarts it.  With the
    counter set just below the wrap, single-token and four-token calls before,
    across and after it give the results of ordinary calls, bitwise."""
    synth, m, ids, w = model
    x = torch.from_numpy(fg.tokens(0, range(900, 904))).cuda()
    ref1 = m.forward(x[:1])
    ref4 = m.forward(x)
    torch.cuda.synchronize()
    with pytest.raises(F.FlintMoEError):
        m.debug_set_epoch(0xFFFFFB80)          # not a multiple of 256
    with pytest.raises(F.FlintMoEError):
        m.debug_set_epoch(256)                 # below the current counter
    m.debug_set_epoch(0xFFFFFB00)
    outs = []
    for i in range(6):                         # counter: ..FC00, ..FD00, ..FE00, wrap -> 256, 512, 768
        outs.append((m.forward(x[:1]) if i % 2 == 0 else m.forward(x), i % 2))
    torch.cuda.synchronize()
    m.status()
    for i, (o, kind) in enumerate(outs):
        assert torch.equal(o, ref4 if kind else ref1), i


def test_persistent_launches_from_two_streams(model):
    """Two handles on two streams, calls queued alternately with no host
    synchronisation: the persistent kernels need every workgroup resident at
    once, so a launch on another stream than the previous one waits for it.
    Each handle's results must equal the same calls run on one stream."""
    synth, m, ids, w = model
    layers = build_layers(synth, range(N_LAYERS))
    m2 = F.FlintMoE(layers)
    del layers
    x = torch.from_numpy(fg.tokens(0, range(800, 816))).cuda()
    calls = [(1, 0, N_LAYERS), (3, 0, 2), (1, 1, N_LAYERS), (9, 0, N_LAYERS), (1, 0, N_LAYERS), (16, 0, N_LAYERS)]
    try:
        torch.cuda.synchronize()
        refs = [m.forward(x[:n].contiguous(), l0, l1) for n, l0, l1 in calls]
        torch.cuda.synchronize()
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        outs = []
        for i, (n, l0, l1) in enumerate(calls):
            for hm, st in ((m, s1), (m2, s2)):
                with torch.cuda.stream(st):
                    outs.append(hm.forward(x[:n].contiguous(), l0, l1, stream=st.cuda_stream))
        torch.cuda.synchronize()
        m.status()
        m2.status()
        for i in range(len(calls)):
            assert torch.equal(outs[2 * i], refs[i]), ("stream 1", i, calls[i])
            assert torch.equal(outs[2 * i + 1], refs[i]), ("stream 2", i, calls[i])
    finally:
        m2.close()
