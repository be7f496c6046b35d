"""Exact rational expansion of the KDA recurrence for tiny cases -- TEST
INFRASTRUCTURE ONLY.

The per-token update of the ogis-ri NLP primer on Kimi K3, §3.1 "KDA", folds
the decay, the erase along k_t and the write into one affine map,
    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T .
Its solution is written out here as explicit products of d_k x d_k matrices,
    S_t = P_(1..t) S0 + sum_{i<=t} P_(i+1..t) beta_i k_i v_i^T,
    P_(a..t) = F_t F_{t-1} ... F_a,   F_s = (I - beta_s k_s k_s^T) Diag(alpha_s),
and o_t = S_t^T q_t, in Python `fractions.Fraction` arithmetic (exact).
Intended for T <= 8 and d <= 4.  It shares no code with the fp64 oracle.

Parity: exact by construction; the fp64 oracle is checked against it.
"""
from __future__ import annotations

from fractions import Fraction


def _eye(n):
    return [[Fraction(int(i == j)) for j in range(n)] for i in range(n)]


def _mm(a, b):
    return [[sum((a[i][p] * b[p][j] for p in range(len(b))), Fraction(0)) for j in range(len(b[0]))]
            for i in range(len(a))]


def _add(a, b):
    return [[a[i][j] + b[i][j] for j in range(len(a[0]))] for i in range(len(a))]


def _outer(x, y, s):
    return [[s * xi * yj for yj in y] for xi in x]


def _transition(k, alpha, beta):
    """F = (I - beta k k^T) Diag(alpha)."""
    n = len(k)
    return [[((Fraction(int(i == j)) - beta * k[i] * k[j]) * alpha[j]) for j in range(n)] for i in range(n)]


def expand(q, k, v, beta, alpha, S0):
    """q, k, alpha: [T][dk]; v: [T][dv]; beta: [T]; S0: [dk][dv] (Fractions).
    Returns (o [T][dv], S_T [dk][dv]) exactly."""
    T = len(q)
    dk, dv = len(k[0]), len(v[0])
    F = [_transition(k[t], alpha[t], beta[t]) for t in range(T)]
    outs = []
    S_t = None
    for t in range(T):
        P = _eye(dk)                        # P = F_t ... F_0
        for s in range(0, t + 1):
            P = _mm(F[s], P)
        S_t = _mm(P, S0)
        for i in range(t + 1):
            Pi = _eye(dk)
            for s in range(i + 1, t + 1):
                Pi = _mm(F[s], Pi)
            S_t = _add(S_t, _mm(Pi, _outer(k[i], v[i], beta[i])))
        outs.append([sum((S_t[c][j] * q[t][c] for c in range(dk)), Fraction(0)) for j in range(dv)])
    if S_t is None:
        S_t = [row[:] for row in S0]
    return outs, S_t
