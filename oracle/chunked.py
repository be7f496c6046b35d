"""Chunkwise fp64 CPU form of the KDA forward pass -- TEST INFRASTRUCTURE ONLY.

A second, independent CPU implementation used to pin the recurrence oracle
(the result must not depend on the chunk size, including chunk 1 and chunk =
whole sequence) and to give stage intermediates (cumulative log-decay, the
triangular system, W, U, corrected values, per-chunk states) for debugging.
It shares no code with `kda_oracle.c` nor with the GPU library.

Source of the form (ogis-ri NLP primer on Kimi K3, §3.1 "KDA"):
  * the sequence is cut into chunks of C tokens; a token's output is the
    read-out of the state carried into its chunk plus an intra-chunk causal
    (i <= j) term;
  * per-channel cumulative decay from the chunk start, Gamma_i; the decay from
    token i to token j is Gamma_j / Gamma_i (§3.1 "chunk 内の減衰と、その数値範囲");
  * the pages say a delta-rule correction enters the intra-chunk term but
    print no formula.  The correction used here is derived by substituting
    the unrolled state into the delta of every token of the chunk: with
    u~_r = beta_r e_r (the written deltas),
        (I + A) U~ = diag(beta) (V - (K . Gamma) S),
        A[r, i]   = beta_r sum_c k_rc k_ic Gamma_rc / Gamma_ic      (i < r)
    then  O  = (Q . Gamma) S + M U~,  M[r, i] = sum_c q_rc k_ic Gamma_rc/Gamma_ic (i <= r)
    and   S' = Diag(Gamma_L) S + (K . Gamma_L / Gamma)^T U~.
The ratios Gamma_r / Gamma_i are formed directly as exp(b_r - b_i) of the
cumulative log-decay b, so no quantity overflows at any chunk size.

Parity: pinned against the recurrence oracle (chunk-size invariance) and the
closed forms in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def forward_chunked(q, k, v, beta, g, S0=None, cu_seqlens=None, chunk=64, stages=False):
    q, k, v, beta, g = (np.asarray(a, dtype=np.float64) for a in (q, k, v, beta, g))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    o = np.zeros((T, H, dv))
    ST = np.zeros((N, H, dk, dv))
    rec = [] if stages else None
    for n in range(N):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[n, h], dtype=np.float64)
            for c0 in range(int(cu[n]), int(cu[n + 1]), chunk):
                c1 = min(c0 + chunk, int(cu[n + 1]))
                Q, K, V, G = q[c0:c1, h], k[c0:c1, h], v[c0:c1, h], g[c0:c1, h]
                Bt = beta[c0:c1, h]
                L = c1 - c0
                b = np.cumsum(G, axis=0)                               # [L, dk]
                causal = np.tril(np.ones((L, L), dtype=bool))          # i <= r
                diff = np.where(causal[:, :, None], b[:, None, :] - b[None, :, :], -np.inf)
                D = np.exp(diff)                                      # decay i -> r per channel
                M = np.einsum("rc,ic,ric->ri", Q, K, D)
                A = Bt[:, None] * np.einsum("rc,ic,ric->ri", K, K, D)
                A = np.tril(A, -1)
                Gam = np.exp(b)
                rhs = Bt[:, None] * (V - (K * Gam) @ S)
                Ut = solve_triangular(np.eye(L) + A, rhs, lower=True, unit_diagonal=True)
                O = (Q * Gam) @ S + M @ Ut
                if stages:
                    Tm = solve_triangular(np.eye(L) + A, np.eye(L), lower=True, unit_diagonal=True)
                    rec.append(dict(seq=n, head=h, start=c0, b=b, A=A, T=Tm,
                                    W=Tm @ (Bt[:, None] * (K * Gam)), U=Tm @ (Bt[:, None] * V),
                                    Ut=Ut, S_in=S.copy(), M=M, O=O))
                o[c0:c1, h] = O
                S = np.exp(b[-1])[:, None] * S + (K * np.exp(b[-1][None, :] - b)).T @ Ut
            ST[n, h] = S
    return (o, ST, rec) if stages else (o, ST)
