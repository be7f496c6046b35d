"""Writes the exact-rational fixtures in this folder.

Calls only `oracle.bruteforce` (exact Fraction arithmetic); run from the repo
root:  python tests/golden/make_golden.py
"""
import json
import os
import sys
from fractions import Fraction

import numpy as np

sys.path.insert(0, os.path.abspath(os.path.join(os.path.dirname(__file__), "..", "..")))
from oracle import bruteforce  # noqa: E402


def _rat(rng, lo, hi, den):
    return Fraction(int(rng.integers(lo * den, hi * den + 1)), den)


def make_case(seed, T, dk, dv, with_s0, beta_one_every=0):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = [[_rat(rng, -1, 1, 8) for _ in range(dk)] for _ in range(T)]
    k = [[_rat(rng, -1, 1, 8) for _ in range(dk)] for _ in range(T)]
    v = [[_rat(rng, -2, 2, 4) for _ in range(dv)] for _ in range(T)]
    beta = [Fraction(int(rng.integers(1, 16)), 16) for _ in range(T)]
    if beta_one_every:
        for t in range(0, T, beta_one_every):
            beta[t] = Fraction(1)
    alpha = [[Fraction(int(rng.integers(1, 32)), 32) for _ in range(dk)] for _ in range(T)]
    S0 = [[(_rat(rng, -1, 1, 16) if with_s0 else Fraction(0)) for _ in range(dv)] for _ in range(dk)]
    o, ST = bruteforce.expand(q, k, v, beta, alpha, S0)
    s = lambda m: [[str(x) for x in row] for row in m]
    return dict(seed=seed, T=T, d_k=dk, d_v=dv, q=s(q), k=s(k), v=s(v), beta=[str(x) for x in beta],
                alpha=s(alpha), S0=s(S0), o=s(o), S_T=s(ST))


if __name__ == "__main__":
    cases = [make_case(1, 6, 3, 2, True), make_case(2, 8, 4, 3, False, beta_one_every=3),
             make_case(3, 7, 4, 4, True, beta_one_every=2)]
    out = dict(source="exact rational expansion S_t = P S0 + sum_i P_(i+1..t) beta_i k_i v_i^T, o_t = S_t^T q_t "
                      "(written by tests/golden/make_golden.py via oracle.bruteforce)",
               cases=cases)
    path = os.path.join(os.path.dirname(__file__), "bruteforce_small.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)
