"""The seeded input generator: reference hash, determinism, distributions."""
import numpy as np
import torch

import flintgen as fg


def test_lowbias32_known_values_and_vectorised_match():
    # scalar reference against a direct transcription of the hash's definition
    def ref(x):
        x &= 0xFFFFFFFF
        x ^= x >> 16
        x = (x * 0x7FEB352D) % 2 ** 32
        x ^= x >> 15
        x = (x * 0x846CA68B) % 2 ** 32
        x ^= x >> 16
        return x
    xs = [0, 1, 2, 0xFFFFFFFF, 0x80000000, 123456789, 0xDEADBEEF]
    rng = np.random.default_rng(0)
    xs += [int(v) for v in rng.integers(0, 2 ** 32, size=2000, dtype=np.uint64)]
    t = fg.lowbias32(torch.tensor(xs, dtype=torch.int64)).tolist()
    assert t == [ref(x) for x in xs] == [fg.lowbias32_int(x) for x in xs]
    assert fg.lowbias32_int(0) == 0


def test_block_words_match_scalar_reference():
    for key in [(0, 0, 0, 0), (0, 46, 2, 255), (7, 3, 12, 9)]:
        w = fg._words([fg.block_key(*key)], 64, "cpu")[0].tolist()
        assert w == [fg.words_int(*key, i) for i in range(64)]


def test_codes_are_uniform_nibbles_little_endian():
    s = fg.Synth(fg.FLINT, 0, 1)
    e = s.experts(0, [5])
    gate = e["gate"][0].numpy()
    assert gate.shape == (512, 1024) and gate.dtype == np.uint8
    # first byte = low byte of word 0 of the (seed 0, layer 0, gate, expert 5) block
    w0 = fg.words_int(0, 0, fg.T_GATE, 5, 0)
    assert gate[0, :4].tolist() == [(w0 >> (8 * i)) & 0xFF for i in range(4)]
    nib = np.concatenate([gate.ravel() & 15, gate.ravel() >> 4])
    counts = np.bincount(nib, minlength=16)
    expect = nib.size / 16
    chi2 = float(((counts - expect) ** 2 / expect).sum())
    assert chi2 < 60, chi2          # 15 dof; p ~ 1e-7 at 60


def test_scales_in_range_and_power_of_two_multiplier():
    s = fg.Synth(fg.FLINT, 0, 1)
    m = fg.Synth(fg.FLINT, 0, 1, up_scale_mult={0: 4096})
    a, b = s.experts(0, [1]), m.experts(0, [1])
    v = a["up_s"].view(torch.bfloat16).double()
    assert float(v.min()) >= 0.005 - 1e-4 and float(v.max()) <= 0.02 + 1e-4
    assert torch.equal(b["up_s"].view(torch.bfloat16).double(), v * 4096)
    assert torch.equal(a["gate_s"], b["gate_s"]) and torch.equal(a["down_s"], b["down_s"])


def test_regenerating_one_expert_matches_whole_layer():
    s = fg.Synth(fg.TINY, 3, 1)
    all_ex = s.experts(0, range(16))
    one = s.experts(0, [9])
    for k in all_ex:
        assert torch.equal(all_ex[k][9], one[k][0])


def test_router_bias_tokens_deterministic():
    s = fg.Synth(fg.FLINT, 0, 2)
    assert s.router(1).dtype == torch.int16 and s.router(1).shape == (256, 2048)
    assert torch.equal(s.router(1), s.router(1)) and not torch.equal(s.router(0), s.router(1))
    w = s.router(0).view(torch.bfloat16).double()
    assert abs(float(w.std()) * np.sqrt(2048) - 1) < 0.02
    b = s.bias(0)
    assert b.dtype == torch.float32 and float(b.abs().max()) < 0.1
    z = fg.Synth(fg.FLINT, 0, 1, bias_kind="zipf").bias(0)
    assert float(z.max()) == 0.0 and abs(float(z.min()) + 0.05 * 1.1 * np.log(256)) < 1e-6
    assert np.array_equal(fg.token(0, 5), fg.token(0, 5))
    assert fg.tokens(0, range(3)).shape == (3, 2048)
