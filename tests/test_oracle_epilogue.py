"""Pins of the epilogue oracle (RMSNorm then a per-channel sigmoid gate, fp64).

Closed forms fix every part of the definition: the mean (not the sum) of
squares over the channels, the square root, eps inside it, the weight, and
the sign and scale of the gate.  A planted-mistake test mutates the
oracle's source and checks that some pin fails for each mutation."""
import math
import os

import numpy as np
import pytest

from oracle import epilogue

SRC = os.path.join(os.path.dirname(epilogue.__file__), "epilogue.py")


def _pins(fn):
    """Runs every pin against `fn`; returns the list of failed pin names."""
    failed = []
    # hand example: o = (3, 4), w = (1, 2), z = (0, ln 3), eps = 0:
    # mean of squares 12.5, so y = (3 / sqrt(12.5) * 1 * 1/2, 4 / sqrt(12.5) * 2 * 3/4)
    y = fn(np.array([3.0, 4.0]), np.array([0.0, math.log(3.0)]), np.array([1.0, 2.0]), 0.0)
    r = math.sqrt(12.5)
    if not np.allclose(y, [1.5 / r, 6.0 / r], rtol=1e-14, atol=0):
        failed.append("hand example")
    rng = np.random.default_rng(3)
    o = rng.standard_normal((5, 3, 64))
    z = rng.standard_normal((5, 3, 64))
    # an open gate (z -> +inf) leaves unit root-mean-square (eps = 0, no weight)
    y = fn(o, np.full_like(o, 60.0), None, 0.0)
    if not np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-13):
        failed.append("unit rms")
    # z = 0 halves the normalised value
    if not np.allclose(fn(o, np.zeros_like(o), None, 0.0), 0.5 * fn(o, np.full_like(o, 60.0), None, 0.0),
                       rtol=1e-13):
        failed.append("half gate")
    # scale invariance without eps; eps matters only against the mean square
    if not np.allclose(fn(7.0 * o, z, None, 0.0), fn(o, z, None, 0.0), rtol=1e-13):
        failed.append("scale invariance")
    small = 1e-4 * o
    ms = np.mean(small * small, axis=-1, keepdims=True)
    want = small / np.sqrt(ms + 1e-6) / (1.0 + np.exp(-z))
    if not np.allclose(fn(small, z, None, 1e-6), want, rtol=1e-12):
        failed.append("eps inside the root")
    # gate symmetry: sigmoid(z) + sigmoid(-z) = 1
    if not np.allclose(fn(o, z, None, 0.0) + fn(o, -z, None, 0.0), fn(o, np.full_like(o, 60.0), None, 0.0),
                       rtol=1e-12):
        failed.append("gate symmetry")
    # the weight multiplies channel by channel
    w = rng.uniform(0.5, 2.0, 64)
    if not np.allclose(fn(o, z, w, 0.0), fn(o, z, None, 0.0) * w, rtol=1e-13):
        failed.append("weight")
    # zero rows stay zero with eps > 0
    if not np.all(fn(np.zeros((2, 64)), np.zeros((2, 64)), None, 1e-6) == 0.0):
        failed.append("zero row")
    return failed


def test_oracle_meets_every_pin():
    assert _pins(epilogue.output_gate) == []


MUTATIONS = [
    ("sum instead of mean", "np.mean(o * o, axis=-1, keepdims=True)", "np.sum(o * o, axis=-1, keepdims=True)"),
    ("no square root", "np.sqrt(mean_sq + eps)", "(mean_sq + eps)"),
    ("eps outside the root", "np.sqrt(mean_sq + eps)", "(np.sqrt(mean_sq) + eps)"),
    ("gate sign", "np.exp(-z)", "np.exp(z)"),
    ("weight dropped", "normed = normed * np.asarray(weight, dtype=np.float64)", "normed = normed"),
    ("mean over the wrong axis", "axis=-1, keepdims=True", "axis=0, keepdims=True"),
]


@pytest.mark.parametrize("what,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistakes_are_caught(what, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, what
    ns = {}
    exec(compile(src.replace(old, new), "mutant", "exec"), ns)
    assert _pins(ns["output_gate"]) != [], what
