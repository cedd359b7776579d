"""Test-side helpers: hand-built layer sources for the oracle pins.

These build inputs only (packing integer codes into bytes, choosing bf16 bit
patterns); none of the block's arithmetic lives here.
"""
import numpy as np
import torch

import flintgen as fg


def pack_codes(v) -> np.ndarray:
    """int [..., K] in [-8, 7] -> uint8 [..., K/2]; even k in the low nibble."""
    v = np.asarray(v, dtype=np.int64)
    assert v.min() >= -8 and v.max() <= 7
    n = (v & 0xF).astype(np.uint8)
    return (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)


def bf16_bits(x) -> np.ndarray:
    """float values -> bf16 bit patterns (int16), round to nearest even (torch)."""
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy()


class ArraySource:
    """One layer's tensors held as NumPy arrays in the canonical layout."""

    def __init__(self, router, bias, experts, shared):
        self._router = np.asarray(router)
        self._bias = np.asarray(bias, dtype=np.float32)
        self._ex = {k: np.asarray(v) for k, v in experts.items()}
        self._sh = {k: np.asarray(v) for k, v in shared.items()}

    def router(self, layer):
        return self._router

    def bias(self, layer):
        return self._bias

    def experts(self, layer, ids):
        ids = [int(i) for i in ids]
        return {k: v[ids] for k, v in self._ex.items()}

    def shared(self, layer):
        return self._sh

    # mutators used by the invariance pins
    def replace(self, router=None, bias=None, experts=None, shared=None):
        return ArraySource(self._router if router is None else router,
                           self._bias if bias is None else bias,
                           self._ex if experts is None else experts,
                           self._sh if shared is None else shared)

    @property
    def ex(self):
        return self._ex

    @property
    def sh(self):
        return self._sh


def synth_source(shape=fg.TINY, seed=0, layer=0, **kw) -> ArraySource:
    """All tensors of one synthetic layer (small shapes only)."""
    s = fg.Synth(shape, seed, layer + 1, **kw)
    ex = {k: v.numpy() for k, v in s.experts(layer, range(shape.n_experts)).items()}
    sh = {k: v.numpy() for k, v in s.shared(layer).items()}
    return ArraySource(s.router(layer).numpy(), s.bias(layer).numpy(), ex, sh)


class SynthSource:
    """Lazy source over a flintgen.Synth: generates only the experts asked for."""

    def __init__(self, synth: fg.Synth):
        self.s = synth

    def router(self, layer):
        return self.s.router(layer).numpy()

    def bias(self, layer):
        return self.s.bias(layer).numpy()

    def experts(self, layer, ids):
        return {k: v.numpy() for k, v in self.s.experts(layer, ids).items()}

    def shared(self, layer):
        return {k: v.numpy() for k, v in self.s.shared(layer).items()}
