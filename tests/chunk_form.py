"""Chunkwise (WY/UT) form of the gated delta rule, fp64 numpy.

Not the oracle and not the GPU path: it writes out, for the CPU tests, the
algebra the chunked kernels implement, so that its exactness against the
token-by-token recurrence is checked on its own. Derived from eq. (5) of
section 2.1.1 by unrolling the recurrence inside one chunk of C tokens:
with G_r the running sum of g = log(alpha) inside the chunk, gamma_r = e^{G_r},
A[r,i] = beta_r e^{G_r - G_i} (k_r . k_i) for i < r, T = (I + A)^{-1}:
    U   = T (diag(beta) V - diag(beta gamma) K S0)
    Y   = diag(gamma) Q S0 + (M o Q K^T) U,     M[r,i] = e^{G_r - G_i} for i <= r
    S_C = gamma_C S0 + (diag(gamma_C / gamma) K)^T U
"""
import numpy as np


def chunked_forward(q, k, v, g, beta, S0=None, cu_seqlens=None, C=64):
    ntok, H, dk = q.shape
    dv = v.shape[2]
    cu = [0, ntok] if cu_seqlens is None else list(cu_seqlens)
    nseq = len(cu) - 1
    y = np.zeros((ntok, H, dv))
    ST = np.zeros((nseq, H, dk, dv))
    for s in range(nseq):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else S0[s, h].copy()
            for c0 in range(cu[s], cu[s + 1], C):
                sl = slice(c0, min(c0 + C, cu[s + 1]))
                Q, K, V = q[sl, h], k[sl, h], v[sl, h]
                G = np.cumsum(g[sl, h])
                b = beta[sl, h]
                n = len(G)
                D = G[:, None] - G[None, :]
                low = np.tril(np.ones((n, n)), -1).astype(bool)
                A = np.where(low, b[:, None] * np.exp(np.where(low, D, 0.0)) * (K @ K.T), 0.0)
                T = np.linalg.inv(np.eye(n) + A)
                gam = np.exp(G)
                U = T @ (b[:, None] * V - (b * gam)[:, None] * (K @ S))
                incl = np.tril(np.ones((n, n))).astype(bool)
                M = np.where(incl, np.exp(np.where(incl, D, 0.0)), 0.0)
                y[sl, h] = gam[:, None] * (Q @ S) + (M * (Q @ K.T)) @ U
                S = gam[-1] * S + (np.exp(G[-1] - G)[:, None] * K).T @ U
            ST[s, h] = S
    return y, ST
