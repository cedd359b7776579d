"""Helpers for GPU-vs-oracle parity: selection rule, error measures, and
building a library handle from seeded synthetic layers."""
import numpy as np

import flintgen as fg

# Expert selection must match the oracle except where the k-th and (k+1)-th
# selection scores differ by less than this (a near tie).
NEAR_TIE = 1e-4
# Relative L2 error bound on each token's block output delta.
REL_L2_SPEC = 2e-3
# Tighter bound from the decode arithmetic: fp32 accumulation of exact
# products over <= 2048 terms, fp32 weights and activations: ~1e-6 observed
# scale; 1e-5 leaves a 10x margin and still fails any dropped or wrong term.
REL_L2_DECODE = 1e-5


def selection_ok(gpu_ids, route, k, tol=NEAR_TIE):
    """True if the GPU's set equals the oracle's, or differs only among
    experts within ``tol`` of the selection boundary."""
    g = set(int(e) for e in gpu_ids)
    if len(g) != k:
        return False
    c = route.c
    ck, ck1 = c[route.order[k - 1]], c[route.order[k]]
    must = set(np.flatnonzero(c > ck1 + tol).tolist())
    allowed = set(np.flatnonzero(c >= ck - tol).tolist())
    return must <= g <= allowed


def rel_l2(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    if den == 0:
        return 0.0 if np.all(got == 0) else np.inf
    return float(np.linalg.norm(got - want) / den)


def build_layers(synth: fg.Synth, layers, device="cuda"):
    """Generate the given layers on ``device`` (canonical layout tensors)."""
    return [synth.layer(l, device) for l in layers]
