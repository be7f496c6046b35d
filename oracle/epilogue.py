"""fp64 CPU oracle of the KDA output epilogue -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may use this module; it shares no code with the GPU library.

What it computes (ogis-ri NLP primer on Kimi K3, §3.1 "KDA", the paragraph
on the output gate): the read-out o_t of every head is normalised by
RMSNorm, because its magnitude varies with the state, and then multiplied
element by element by a per-channel value in (0, 1) made from the layer
input x_t; the output projection W_o follows and is not part of it.  The
printed formula did not survive extraction; the reading taken here:

    y_t = RMSNorm(o_t) * sigmoid(z_t),   RMSNorm(x) = x / sqrt(mean(x^2) + eps) * w

per (token, head), the mean taken over the head's d_v channels, w an
optional per-channel weight (ones when absent), and z_t the gate's
pre-activation (the projection of x_t, computed outside).  sigmoid maps
z_t to (0, 1) as the pages require.

Parity: pinned by closed forms in tests/test_oracle_epilogue.py.
"""
from __future__ import annotations

import numpy as np


def output_gate(o, z, weight=None, eps=1e-6):
    """o, z: [..., d_v] (any float dtype); weight: [d_v] or None.  Returns fp64."""
    o = np.asarray(o, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    assert o.shape == z.shape
    mean_sq = np.mean(o * o, axis=-1, keepdims=True)
    normed = o / np.sqrt(mean_sq + eps)
    if weight is not None:
        normed = normed * np.asarray(weight, dtype=np.float64)
    return normed * (1.0 / (1.0 + np.exp(-z)))
