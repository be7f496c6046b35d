"""Pins of the oracle's backward pass (reverse-mode derivative of the KDA
recurrence, fp64, CPU).

The gradient is pinned to the forward oracle by central finite differences
of a scalar loss L = sum(dO * o) + sum(dS_T * S_T), element by element over
every input (q, k, v, beta, log alpha, S0), on varlen batches with an empty
sequence and with / without final-state gradients.  Mistakes planted in the
backward source (dropped terms, flipped signs, a missing decay factor) are
each caught by that pin.
"""
import numpy as np
import pytest

import oracle


def _case(seed, lengths, H, dk, dv):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    g = -5.0 / (1.0 + np.exp(-2.0 * rng.standard_normal((T, H, dk))))
    N = len(lengths)
    S0 = rng.standard_normal((N, H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    dO = rng.standard_normal((T, H, dv))
    dST = rng.standard_normal((N, H, dk, dv))
    return dict(q=q, k=k, v=v, beta=beta, g=g, S0=S0, cu=cu, dO=dO, dST=dST)


NAMES = (("q", "dq"), ("k", "dk"), ("v", "dv"), ("beta", "dbeta"), ("g", "dg"), ("S0", "dS0"))


def _fd_error(c, grads, fwd=oracle.forward, use_dst=True, h=1e-6):
    dST = c["dST"] if use_dst else np.zeros_like(c["dST"])

    def loss(x):
        o, ST = fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], x["S0"], c["cu"])
        return float((o * c["dO"]).sum() + (ST * dST).sum())

    worst = 0.0
    for name, gname in NAMES:
        arr = c[name]
        for idx in np.ndindex(arr.shape):
            xp = dict(c)
            xm = dict(c)
            xp[name] = arr.copy()
            xm[name] = arr.copy()
            xp[name][idx] += h
            xm[name][idx] -= h
            fd = (loss(xp) - loss(xm)) / (2 * h)
            worst = max(worst, abs(fd - grads[gname][idx]) / max(1.0, abs(fd)))
    return worst


@pytest.mark.parametrize("lengths,H,dk,dv,use_dst", [([5, 4], 2, 4, 3, True), ([7, 0, 3], 1, 3, 5, False),
                                                     ([70], 1, 2, 2, True)],
                         ids=["varlen", "empty-seq-no-dST", "two-blocks"])
def test_backward_matches_finite_differences(lengths, H, dk, dv, use_dst):
    c = _case(sum(lengths) + dk, lengths, H, dk, dv)
    grads = oracle.backward(c["q"], c["k"], c["v"], c["beta"], c["g"], c["dO"], c["S0"],
                            c["dST"] if use_dst else None, c["cu"])
    err = _fd_error(c, grads, use_dst=use_dst)
    assert err < 1e-6, err


def test_backward_empty_sequence_passes_state_gradient():
    c = _case(3, [4, 0], 1, 3, 2)
    grads = oracle.backward(c["q"], c["k"], c["v"], c["beta"], c["g"], c["dO"], c["S0"], c["dST"], c["cu"])
    assert np.array_equal(grads["dS0"][1], c["dST"][1])    # S_T = S0 for an empty sequence


def test_backward_is_linear_in_output_gradients():
    c = _case(4, [6, 5], 2, 3, 4)
    a = oracle.backward(c["q"], c["k"], c["v"], c["beta"], c["g"], c["dO"], c["S0"], c["dST"], c["cu"])
    b = oracle.backward(c["q"], c["k"], c["v"], c["beta"], c["g"], 2.0 * c["dO"], c["S0"], 2.0 * c["dST"], c["cu"])
    for _, gname in NAMES:
        np.testing.assert_allclose(b[gname], 2.0 * a[gname], rtol=1e-12, atol=1e-12)


PLANTS = [
    ("dk drops -P de", "dk[(t * n_heads + h) * d_k + i] = bt * ge - pde;", "dk[(t * n_heads + h) * d_k + i] = bt * ge;"),
    ("dP sign", "const double dp = G[i * d_v + j] - kt[i] * de[j];", "const double dp = G[i * d_v + j] + kt[i] * de[j];"),
    ("no decay on G", "G[i * d_v + j] = alpha[i] * dp;", "G[i * d_v + j] = dp;"),
    ("dg without alpha", "dg[(t * n_heads + h) * d_k + i] = alpha[i] * s;", "dg[(t * n_heads + h) * d_k + i] = s;"),
    ("dv without beta", "de[j] = bt * gk;", "de[j] = gk;"),
    ("dq from S_{t-1}", "s += Scur[i * d_v + j] * dot[j];", "s += Sprev[i * d_v + j] * dot[j];"),
]


@pytest.mark.parametrize("what,old,new", PLANTS, ids=[p[0] for p in PLANTS])
def test_planted_backward_mistakes_are_caught(tmp_path, what, old, new):
    src = oracle.source_text()
    assert src.count(old) == 1, what
    fwd = oracle.compile_variant(src.replace(old, new), str(tmp_path / "variant.so"))
    c = _case(9, [4, 3], 1, 3, 2)
    grads = fwd.backward(c["q"], c["k"], c["v"], c["beta"], c["g"], c["dO"], c["S0"], c["dST"], c["cu"])
    assert _fd_error(c, grads) > 1e-4, what


@pytest.mark.parametrize("lengths,chunk", [([37, 20], 16), ([70], 64), ([5, 0, 9], 4), ([130], 64)],
                         ids=["varlen-c16", "one-c64", "empty-c4", "three-chunks-c64"])
def test_chunked_backward_matches_recurrence_backward(lengths, chunk):
    """The chunk-level backward algebra (the form the GPU backward follows)
    gives the recurrence oracle's gradients to rounding, at any chunk size."""
    from oracle import chunked
    c = _case(sum(lengths) + chunk, lengths, 2, 8, 6)
    ref = oracle.backward(c["q"], c["k"], c["v"], c["beta"], c["g"], c["dO"], c["S0"], c["dST"], c["cu"])
    got = chunked.backward_chunked(c["q"], c["k"], c["v"], c["beta"], c["g"], c["dO"], c["S0"], c["dST"],
                                   c["cu"], chunk=chunk)
    for _, gname in NAMES:
        err = np.max(np.abs(got[gname] - ref[gname])) / max(1e-30, np.max(np.abs(ref[gname])))
        assert err < 1e-12, (gname, err)
