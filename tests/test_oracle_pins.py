"""Pins for the fp64 oracle: closed forms, invariants, special cases and exact
brute force, each independent of the recurrence code it checks.

Every pin is a function `pin_*(fwd)` taking a forward() callable, so the
planted-mistake test at the bottom can run the same pins on deliberately
broken copies of the oracle and show each mistake is caught.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import chunked

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(lengths, H, dk, dv, seed, s0=0.3, g_scale=1.0):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    q = rng.standard_normal((T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    g = g_scale * (-5.0 / (1.0 + np.exp(-2.0 * rng.standard_normal((T, H, dk)))))
    N = len(lengths)
    S0 = s0 * rng.standard_normal((N, H, dk, dv)) if s0 else None
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return q, k, v, beta, g, S0, cu


def _close(a, b, tol, what=""):
    a, b = np.asarray(a), np.asarray(b)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) / scale if a.size else 0.0
    assert err <= tol, "%s: max err %.3e > %.1e" % (what, err, tol)


# ---------------------------------------------------------------- pins
def pin_beta_zero(fwd):
    """beta = 0: nothing is written or erased, only decayed.
    o_t = S0^T (q_t . exp(sum_{s<=t} g_s)),  S_T = Diag(exp(sum g)) S0."""
    q, k, v, beta, g, S0, cu = _case([23, 9], 2, 6, 5, seed=1)
    beta[:] = 0.0
    o, ST = fwd(q, k, v, beta, g, S0, cu)
    for n in range(2):
        a, b = cu[n], cu[n + 1]
        G = np.exp(np.cumsum(g[a:b], axis=0))                    # [L, H, dk]
        for h in range(2):
            want = (q[a:b, h] * G[:, h]) @ S0[n, h]
            _close(o[a:b, h], want, 1e-13, "o beta=0")
            _close(ST[n, h], G[-1, h][:, None] * S0[n, h], 1e-13, "S_T beta=0")


def _disjoint_keys(T, H, dk, rng):
    k = np.zeros((T, H, dk))
    for h in range(H):
        chans = rng.permutation(dk)[:T]
        k[np.arange(T), h, chans] = rng.uniform(0.5, 1.5, T) * rng.choice([-1, 1], T)
    return k


def pin_disjoint_keys_gla(fwd):
    """Keys with pairwise disjoint channel support and S0 = 0: the probe
    always returns 0, so KDA is exactly per-channel gated linear attention,
    o_t = sum_{i<=t} beta_i sum_c q_tc k_ic exp(b_tc - b_ic) v_i."""
    rng = np.random.default_rng(2)
    T, H, dk, dv = 12, 2, 16, 3
    q, _, v, beta, g, _, cu = _case([T], H, dk, dv, seed=3, s0=0)
    k = _disjoint_keys(T, H, dk, rng)
    o, ST = fwd(q, k, v, beta, g, None, cu)
    b = np.cumsum(g, axis=0)
    for h in range(H):
        for t in range(T):
            want = np.zeros(dv)
            for i in range(t + 1):
                want += beta[i, h] * np.sum(q[t, h] * k[i, h] * np.exp(b[t, h] - b[i, h])) * v[i, h]
            _close(o[t, h], want, 1e-13, "o GLA")
        Swant = sum(beta[i, h] * np.outer(k[i, h] * np.exp(b[-1, h] - b[i, h]), v[i, h]) for i in range(T))
        _close(ST[0, h], Swant, 1e-13, "S_T GLA")


def pin_disjoint_keys_no_decay(fwd):
    """As above with alpha = 1: cumulative k v^T, o_t = sum_{i<=t} beta_i (q_t.k_i) v_i."""
    rng = np.random.default_rng(4)
    T, H, dk, dv = 10, 1, 12, 4
    q, _, v, beta, g, _, cu = _case([T], H, dk, dv, seed=5, s0=0)
    k = _disjoint_keys(T, H, dk, rng)
    g[:] = 0.0
    o, _ = fwd(q, k, v, beta, g, None, cu)
    for t in range(T):
        want = sum(beta[i, 0] * np.dot(q[t, 0], k[i, 0]) * v[i, 0] for i in range(t + 1))
        _close(o[t, 0], want, 1e-13, "o cumulative kv")


def pin_small_beta_limit(fwd):
    """Generic keys, S0 = 0: o(eps*beta)/eps -> gated linear attention as eps -> 0
    (the erase term is second order in beta)."""
    q, k, v, beta, g, _, cu = _case([40], 1, 8, 5, seed=6, s0=0)
    eps = 1e-7
    o, _ = fwd(q, k, v, eps * beta, g, None, cu)
    b = np.cumsum(g, axis=0)
    want = np.zeros_like(o)
    for t in range(40):
        for i in range(t + 1):
            want[t, 0] += beta[i, 0] * np.sum(q[t, 0] * k[i, 0] * np.exp(b[t, 0] - b[i, 0])) * v[i, 0]
    _close(o / eps, want, 1e-5, "small-beta limit")


def pin_single_token(fwd):
    """One token, S0 = 0: o = beta (q.k) v and S_1 = beta k v^T."""
    q, k, v, beta, g, _, cu = _case([1], 3, 7, 4, seed=7, s0=0)
    o, ST = fwd(q, k, v, beta, g, None, cu)
    for h in range(3):
        _close(o[0, h], beta[0, h] * np.dot(q[0, h], k[0, h]) * v[0, h], 1e-14, "single o")
        _close(ST[0, h], beta[0, h] * np.outer(k[0, h], v[0, h]), 1e-14, "single S")


def pin_replace(fwd):
    """beta = 1, q_t = k_t, |k_t| = 1: the write replaces the value stored
    under k_t, so reading with k_t returns v_t exactly, for any decay and S0."""
    q, k, v, beta, g, S0, cu = _case([30, 17], 2, 8, 6, seed=8, s0=0.7)
    beta[:] = 1.0
    o, _ = fwd(k, k, v, beta, g, S0, cu)
    _close(o, v, 1e-12, "replace")


def pin_linearity(fwd):
    """o and S_T are jointly linear in (S0, V), and o is linear in q."""
    q, k, v, beta, g, S0, cu = _case([50, 21], 2, 8, 6, seed=9)
    rng = np.random.default_rng(10)
    v2 = rng.standard_normal(v.shape)
    S02 = rng.standard_normal(S0.shape)
    q2 = rng.standard_normal(q.shape)
    a, c = 0.7, -1.3
    o1, S1 = fwd(q, k, v, beta, g, S0, cu)
    o2, S2 = fwd(q, k, v2, beta, g, S02, cu)
    o3, S3 = fwd(q, k, a * v + c * v2, beta, g, a * S0 + c * S02, cu)
    _close(o3, a * o1 + c * o2, 1e-12, "linear o in (S0,V)")
    _close(S3, a * S1 + c * S2, 1e-12, "linear S_T in (S0,V)")
    o4, _ = fwd(q2, k, v, beta, g, S0, cu)
    o5, _ = fwd(a * q + c * q2, k, v, beta, g, S0, cu)
    _close(o5, a * o1 + c * o4, 1e-12, "linear o in q")


def pin_composition(fwd):
    """Running [0, t) then [t, T) from S_t equals running [0, T)."""
    q, k, v, beta, g, S0, cu = _case([90], 2, 8, 5, seed=11)
    o, ST = fwd(q, k, v, beta, g, S0, cu)
    t = 37
    oa, Sa = fwd(q[:t], k[:t], v[:t], beta[:t], g[:t], S0, None)
    ob, Sb = fwd(q[t:], k[t:], v[t:], beta[t:], g[t:], Sa, None)
    _close(np.concatenate([oa, ob]), o, 1e-13, "composition o")
    _close(Sb, ST, 1e-13, "composition S")


def pin_transition(fwd):
    """S_T = P S0 + Z, with P the explicit product of the per-token maps
    (I - beta k k^T) Diag(alpha) and Z the zero-start final state."""
    q, k, v, beta, g, S0, cu = _case([25], 1, 6, 4, seed=12)
    _, ST = fwd(q, k, v, beta, g, S0, cu)
    _, Z = fwd(q, k, v, beta, g, None, cu)
    P = np.eye(6)
    for t in range(25):
        F = (np.eye(6) - beta[t, 0] * np.outer(k[t, 0], k[t, 0])) @ np.diag(np.exp(g[t, 0]))
        P = F @ P
    _close(ST[0, 0], P @ S0[0, 0] + Z[0, 0], 1e-13, "transition")


def pin_chunk_invariance(fwd):
    """The independent chunkwise CPU form gives the same result for every
    chunk size, including 1 and the whole sequence; 25 % of channels sit at
    the g = -5 bound."""
    lengths = [37, 200, 19]
    q, k, v, beta, g, S0, cu = _case(lengths, 2, 16, 12, seed=13)
    g[:, :, :4] = -5.0
    o, ST = fwd(q, k, v, beta, g, S0, cu)
    for C in (1, 16, 32, 64, 128, 200):
        oc, Sc = chunked.forward_chunked(q, k, v, beta, g, S0, cu, chunk=C)
        _close(oc, o, 1e-12, "chunked C=%d o" % C)
        _close(Sc, ST, 1e-12, "chunked C=%d S" % C)


def pin_bruteforce_golden(fwd):
    """Exact rational expansion (tests/golden/bruteforce_small.json) vs fp64."""
    with open(os.path.join(GOLDEN, "bruteforce_small.json")) as f:
        gold = json.load(f)
    for c in gold["cases"]:
        F = lambda m: np.array([[float(Fraction(x)) for x in row] for row in m])
        T = c["T"]
        q, k, v, alpha = F(c["q"]), F(c["k"]), F(c["v"]), F(c["alpha"])
        beta = np.array([float(Fraction(x)) for x in c["beta"]])
        S0 = F(c["S0"])
        o, ST = fwd(q[:, None], k[:, None], v[:, None], beta[:, None], np.log(alpha)[:, None],
                    S0[None, None], None)
        _close(o[:, 0], F(c["o"]), 1e-12, "brute force o (seed %d)" % c["seed"])
        _close(ST[0, 0], F(c["S_T"]), 1e-12, "brute force S (seed %d)" % c["seed"])


PINS = [pin_beta_zero, pin_disjoint_keys_gla, pin_disjoint_keys_no_decay, pin_small_beta_limit,
        pin_single_token, pin_replace, pin_linearity, pin_composition, pin_transition,
        pin_chunk_invariance, pin_bruteforce_golden]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(oracle.forward)


def test_bruteforce_fresh_small():
    """A freshly drawn exact case (not from the fixture), d_k = d_v = 2."""
    from oracle import bruteforce
    rng = np.random.default_rng(99)
    T, d = 5, 2
    R = lambda lo, hi, den: Fraction(int(rng.integers(lo * den, hi * den + 1)), den)
    q = [[R(-1, 1, 4) for _ in range(d)] for _ in range(T)]
    k = [[R(-1, 1, 4) for _ in range(d)] for _ in range(T)]
    v = [[R(-1, 1, 4) for _ in range(d)] for _ in range(T)]
    beta = [Fraction(int(rng.integers(1, 9)), 8) for _ in range(T)]
    alpha = [[Fraction(int(rng.integers(1, 9)), 8) for _ in range(d)] for _ in range(T)]
    S0 = [[R(-1, 1, 4) for _ in range(d)] for _ in range(d)]
    o_ex, S_ex = bruteforce.expand(q, k, v, beta, alpha, S0)
    f = lambda m: np.array([[float(x) for x in row] for row in m])
    o, ST = oracle.forward(f(q)[:, None], f(k)[:, None], f(v)[:, None],
                           np.array([float(b) for b in beta])[:, None], np.log(f(alpha))[:, None],
                           f(S0)[None, None], None)
    _close(o[:, 0], f(o_ex), 1e-13, "fresh brute force o")
    _close(ST[0, 0], f(S_ex), 1e-13, "fresh brute force S")


def test_bound_constants():
    """The bounded-decay numbers the pages print (tests/golden/bound_constants.json)."""
    with open(os.path.join(GOLDEN, "bound_constants.json")) as f:
        ent = {e["name"]: e for e in json.load(f)["entries"]}
    g_min = ent["g_lower_bound"]["value"]
    tile = ent["tile_tokens"]["value"]
    assert math.isclose(math.exp(g_min), ent["alpha_min_approx"]["value"], rel_tol=ent["alpha_min_approx"]["rel_tol"])
    lo, hi = ent["tile_logdecay_range"]["value"]
    assert tile * g_min == lo and hi == 0.0
    inv = math.exp(-lo)
    assert math.isclose(inv, ent["inverse_decay_bound_approx"]["value"], rel_tol=0.01)
    bf16_max = float(np.array([0x7F7F0000], dtype=np.uint32).view(np.float32)[0])
    assert math.isclose(bf16_max, ent["bf16_max_approx"]["value"], rel_tol=0.01)
    assert inv < bf16_max                                  # inverse decay of a full tile fits bf16
    bf16_min_normal = float(np.array([0x00800000], dtype=np.uint32).view(np.float32)[0])
    assert math.exp(lo) > bf16_min_normal                 # and so does the decay itself
    assert math.exp(2 * tile * -g_min) > bf16_max         # a 32-token tile would overflow


def test_chunked_stages_consistent():
    """Stage intermediates of the chunked form satisfy their defining identities."""
    q, k, v, beta, g, S0, cu = _case([70], 1, 8, 6, seed=14)
    _, _, rec = chunked.forward_chunked(q, k, v, beta, g, S0, cu, chunk=32, stages=True)
    for r in rec:
        L = r["A"].shape[0]
        _close((np.eye(L) + r["A"]) @ r["T"], np.eye(L), 1e-12, "(I+A)T = I")
        _close(r["Ut"], r["U"] - r["W"] @ r["S_in"], 1e-12, "U~ = U - W S")


# ------------------------------------------------- planted mistakes (CPU only)
MUTATIONS = {
    "no_decay": ("S[i * COLS + j] *= alpha[i];", "S[i * COLS + j] *= 1.0;"),
    "decay_sign": ("alpha[i] = exp(gt[i]);", "alpha[i] = exp(-gt[i]);"),
    "delta_sign": ("e[j] = vt[j] - vhat[j];", "e[j] = vt[j] + vhat[j];"),
    "no_erase": ("e[j] = vt[j] - vhat[j];", "e[j] = vt[j];"),
    "no_beta": ("+= bt * kt[i] * e[j];", "+= kt[i] * e[j];"),
    "probe_with_q": ("vhat[j] += S[i * COLS + j] * kt[i];", "vhat[j] += S[i * COLS + j] * qt[i];"),
    "read_with_k": ("ot[j] += S[i * COLS + j] * qt[i];", "ot[j] += S[i * COLS + j] * kt[i];"),
    "beta_index": ("beta[t * n_heads + h]", "beta[t * n_heads]"),
    "s0_transposed": ("S0[((n * n_heads + h) * d_k + i) * d_v + c0 + j]",
                      "S0[((n * n_heads + h) * d_v + c0 + j) * d_k + i]"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = oracle.source_text()
    # plant in the forward recurrence only (the backward follows it in the file)
    cut = src.index("int kda_oracle_backward(")
    fwd_src, rest = src[:cut], src[cut:]
    assert fwd_src.count(old) == 1, name
    fwd = oracle.compile_variant(fwd_src.replace(old, new) + rest, str(tmp_path / ("oracle_%s.so" % name)))
    caught = []
    for pin in PINS:
        try:
            pin(fwd)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "planted mistake %s passed every pin" % name


def test_parity_metric():
    """max|x - ref| / max|ref| per (sequence, head) slice, with an absolute
    floor for references that decayed to nothing."""
    ref = np.zeros((6, 2, 3))
    ref[:4, 0] = 2.0
    ref[4:, 0] = 10.0
    ref[:, 1] = 1e-300
    x = ref.copy()
    x[1, 0, 0] += 0.2            # seq 0 head 0: 0.2 / 2
    x[5, 0, 2] -= 0.5            # seq 1 head 0: 0.5 / 10
    x[:, 1] = 0.0                # decayed-to-nothing head: absolute
    assert math.isclose(oracle.parity_error(x, ref, [0, 4, 6]), 0.1)
    assert math.isclose(oracle.parity_error(x, ref, None), 0.5 / 10)
    S = np.ones((2, 2, 3, 3))
    S2 = S.copy()
    S2[1, 1, 2, 2] = 1.03
    assert math.isclose(oracle.parity_error(S2, S), 0.03, rel_tol=1e-9)


def test_parity_metric_rejects_nonfinite():
    ref = np.ones((4, 1, 2))
    x = ref.copy()
    x[2, 0, 1] = np.nan
    assert oracle.parity_error(x, ref) == float("inf")
    x[2, 0, 1] = np.inf
    assert oracle.parity_error(x, ref) == float("inf")
