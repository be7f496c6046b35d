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


def backward_chunked(q, k, v, beta, g, dO, S0=None, dS_T=None, cu_seqlens=None, chunk=64):
    """Chunkwise fp64 form of the backward pass -- the algebra the GPU
    backward follows, pinned here against the recurrence oracle's gradients.

    Per chunk (incoming state S, output gradients dO, gradient dS' of the
    outgoing state), with the forward quantities above (b, Gamma, gamma =
    Gamma_L, A, M, T, Y = V - (K.Gamma) S, Z = diag(beta) Y, U~ = T Z,
    K^ = K . exp(b_L - b)) the adjoints are:
        dU~ = M^T dO + K^ dS'
        dZ  = T^T dU~,  dY = diag(beta) dZ,  dV = dY
        dS  = Diag(gamma) dS' + (Q.Gamma)^T dO - (K.Gamma)^T dY
        d(Q.Gamma) = dO S^T,  d(K.Gamma) = -dY S^T,  dK^ = U~ dS'^T
        dgamma_c = sum_j dS'_cj S_cj
        dA = -T^T (dU~ Z^T) T^T  on the strict lower triangle
        dbeta_r = sum_j dZ_rj Y_rj + sum_{i<r} dA_ri A_ri / beta_r
        dGk = diag(beta) dA (strict lower),  dGq = dO U~^T (lower incl. diagonal)
    where Gk, Gq are the decayed Gram matrices sum_c x_rc k_ic exp(b_rc - b_ic).
    Their gradients reach q, k and b element by element; b = cumsum(g)
    makes dg the reverse cumulative sum of db.  Chunks are walked last to
    first, dS' of a chunk being dS of the next one; returns the same dict as
    oracle.backward."""
    q, k, v, beta, g, dO = (np.asarray(a, dtype=np.float64) for a in (q, k, v, beta, g, dO))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    out = dict(dq=np.zeros((T, H, dk)), dk=np.zeros((T, H, dk)), dv=np.zeros((T, H, dv)),
               dbeta=np.zeros((T, H)), dg=np.zeros((T, H, dk)), dS0=np.zeros((N, H, dk, dv)))
    for n in range(N):
        for h in range(H):
            # forward sweep: incoming state of every chunk
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[n, h], dtype=np.float64)
            starts = list(range(int(cu[n]), int(cu[n + 1]), chunk))
            S_in = []
            for c0 in starts:
                c1 = min(c0 + chunk, int(cu[n + 1]))
                S_in.append(S.copy())
                f = _chunk_quantities(q[c0:c1, h], k[c0:c1, h], v[c0:c1, h], beta[c0:c1, h], g[c0:c1, h], S)
                S = f["S_out"]
            dS = np.zeros((dk, dv)) if dS_T is None else np.array(dS_T[n, h], dtype=np.float64)
            for c0, S in zip(reversed(starts), reversed(S_in)):
                c1 = min(c0 + chunk, int(cu[n + 1]))
                Q, K, V, Bt, G = q[c0:c1, h], k[c0:c1, h], v[c0:c1, h], beta[c0:c1, h], g[c0:c1, h]
                f = _chunk_quantities(Q, K, V, Bt, G, S)
                dOc = dO[c0:c1, h]
                L = c1 - c0
                Tm, Z, Y, Ut, Mm, Am, D = f["T"], f["Z"], f["Y"], f["Ut"], f["M"], f["A"], f["D"]
                Gam, Kg, Qg, Kh, gam = f["Gam"], f["Kg"], f["Qg"], f["Kh"], f["gam"]
                dUt = Mm.T @ dOc + Kh @ dS
                dZ = Tm.T @ dUt
                dY = Bt[:, None] * dZ
                dSin = gam[:, None] * dS + Qg.T @ dOc - Kg.T @ dY
                dQg = dOc @ S.T
                dKg = -dY @ S.T
                dKh = Ut @ dS.T
                dgam = np.sum(dS * S, axis=1)
                dA = np.tril(-Tm.T @ (dUt @ Z.T) @ Tm.T, -1)
                Gk = np.einsum("rc,ic,ric->ri", K, K, D)
                dbeta = np.sum(dZ * Y, axis=1) + np.sum(dA * np.tril(Gk, -1), axis=1)
                dGk = Bt[:, None] * dA
                dGq = np.tril(dOc @ Ut.T)
                # decayed-Gram gradients, element by element over channels
                dKr = np.einsum("ri,ic,ric->rc", dGk, K, D)           # k as row operand
                dKc = np.einsum("ri,rc,ric->ic", dGk, K, D)           # k as column operand
                dQr = np.einsum("ri,ic,ric->rc", dGq, K, D)
                dKc += np.einsum("ri,rc,ric->ic", dGq, Q, D)
                db = K * dKr - K * dKc + Q * dQr                       # d/db_r of e^{b_r}, d/db_i of e^{-b_i}
                # Q.Gamma, K.Gamma, K^ and gamma
                dq_c = dQr + dQg * Gam
                dk_c = dKr + dKc + dKg * Gam + dKh * np.exp(f["b"][-1][None, :] - f["b"])
                db += dQg * Qg + dKg * Kg - dKh * Kh
                dbL = np.sum(dKh * Kh, axis=0) + dgam * gam
                db[L - 1] += dbL
                dg_c = np.cumsum(db[::-1], axis=0)[::-1]
                out["dq"][c0:c1, h] = dq_c
                out["dk"][c0:c1, h] = dk_c
                out["dv"][c0:c1, h] = dY
                out["dbeta"][c0:c1, h] = dbeta
                out["dg"][c0:c1, h] = dg_c
                dS = dSin
            out["dS0"][n, h] = dS
    return out


def _chunk_quantities(Q, K, V, Bt, G, S):
    """Forward quantities of one chunk from its incoming state S (fp64)."""
    L = Q.shape[0]
    b = np.cumsum(G, axis=0)
    causal = np.tril(np.ones((L, L), dtype=bool))
    D = np.exp(np.where(causal[:, :, None], b[:, None, :] - b[None, :, :], -np.inf))   # e^{b_r - b_i}, i <= r
    M = np.einsum("rc,ic,ric->ri", Q, K, D)
    A = np.tril(Bt[:, None] * np.einsum("rc,ic,ric->ri", K, K, D), -1)
    Tm = solve_triangular(np.eye(L) + A, np.eye(L), lower=True, unit_diagonal=True)
    Gam = np.exp(b)
    Kg, Qg = K * Gam, Q * Gam
    Y = V - Kg @ S
    Z = Bt[:, None] * Y
    Ut = Tm @ Z
    gam = Gam[-1]
    Kh = K * np.exp(b[-1][None, :] - b)
    S_out = gam[:, None] * S + Kh.T @ Ut
    return dict(b=b, D=D, M=M, A=A, T=Tm, Gam=Gam, Kg=Kg, Qg=Qg, Y=Y, Z=Z, Ut=Ut, gam=gam, Kh=Kh, S_out=S_out)
