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


def chunked_backward(q, k, v, g, beta, dy, S0=None, dST=None, cu_seqlens=None, C=64):
    """Reverse-mode derivative of chunked_forward, chunk by chunk in reverse order, from the
    state at each chunk start (recomputed by a forward sweep). Per chunk, with
    KS = K S, R = beta o (V - gamma o KS), U = T R, W = w o U (w_r = e^{G_C - G_r}),
    Y = gamma o (Q S) + P U and S' = gamma_C S + K^T W, the adjoints are taken in the
    reverse order of those products. Returns dict(dq, dk, dv, dg, dbeta, dS0)."""
    ntok, H, dk = q.shape
    dv = v.shape[2]
    cu = [0, ntok] if cu_seqlens is None else list(cu_seqlens)
    nseq = len(cu) - 1
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               dg=np.zeros_like(g), dbeta=np.zeros_like(beta), dS0=np.zeros((nseq, H, dk, dv)))
    for s in range(nseq):
        for h in range(H):
            starts = list(range(cu[s], cu[s + 1], C))
            S = np.zeros((dk, dv)) if S0 is None else S0[s, h].copy()
            Sc = []
            for c0 in starts:                      # forward: the state at each chunk start
                Sc.append(S.copy())
                sl = slice(c0, min(c0 + C, cu[s + 1]))
                _, S = _chunk_fwd(q[sl, h], k[sl, h], v[sl, h], g[sl, h], beta[sl, h], S)
            dS = np.zeros((dk, dv)) if dST is None else dST[s, h].copy()
            for c0, S in zip(reversed(starts), reversed(Sc)):
                sl = slice(c0, min(c0 + C, cu[s + 1]))
                grads, dS = _chunk_bwd(q[sl, h], k[sl, h], v[sl, h], g[sl, h], beta[sl, h], S,
                                       dy[sl, h], dS)
                for key in ("dq", "dk", "dv"):
                    out[key][sl, h] = grads[key]
                out["dg"][sl, h] = grads["dg"]
                out["dbeta"][sl, h] = grads["dbeta"]
            out["dS0"][s, h] = dS
    return out


def _chunk_parts(Q, K, V, g, b, S):
    n = len(g)
    G = np.cumsum(g)
    D = G[:, None] - G[None, :]
    low = np.tril(np.ones((n, n)), -1).astype(bool)
    incl = np.tril(np.ones((n, n))).astype(bool)
    EA = np.where(low, np.exp(np.where(low, D, 0.0)), 0.0)
    EP = np.where(incl, np.exp(np.where(incl, D, 0.0)), 0.0)
    KK, QK = K @ K.T, Q @ K.T
    A = b[:, None] * EA * KK
    T = np.linalg.inv(np.eye(n) + A)
    gam = np.exp(G)
    KS = K @ S
    R = b[:, None] * (V - gam[:, None] * KS)
    U = T @ R
    P = EP * QK
    w = np.exp(G[-1] - G)
    return dict(G=G, EA=EA, EP=EP, KK=KK, QK=QK, A=A, T=T, gam=gam, KS=KS, R=R, U=U, P=P, w=w,
                low=low, incl=incl)


def _chunk_fwd(Q, K, V, g, b, S):
    p = _chunk_parts(Q, K, V, g, b, S)
    Y = p["gam"][:, None] * (Q @ S) + p["P"] @ p["U"]
    S1 = p["gam"][-1] * S + K.T @ (p["w"][:, None] * p["U"])
    return Y, S1


def _chunk_bwd(Q, K, V, g, b, S, dY, dS1):
    p = _chunk_parts(Q, K, V, g, b, S)
    gam, w, U, R, KS, T = p["gam"], p["w"], p["U"], p["R"], p["KS"], p["T"]
    n = len(g)
    W = w[:, None] * U
    # S' = gamma_C S + K^T W
    dS = gam[-1] * dS1
    dgamC = np.sum(S * dS1)
    dK = W @ dS1.T
    dW = K @ dS1
    # W = w o U
    dU = w[:, None] * dW
    dw = np.sum(dW * U, axis=1)
    # Y = gamma o (Q S) + P U
    QS = Q @ S
    dQ = gam[:, None] * (dY @ S.T)
    dS = dS + Q.T @ (gam[:, None] * dY)
    dgam = np.sum(dY * QS, axis=1)
    dP = np.where(p["incl"], dY @ U.T, 0.0)
    dU = dU + p["P"].T @ dY
    # U = T R
    dR = T.T @ dU
    dA = np.where(p["low"], -dR @ U.T, 0.0)
    # R = b o (V - gamma o KS)
    dV = b[:, None] * dR
    db = np.sum(dR * (V - gam[:, None] * KS), axis=1)
    dKS = -(b * gam)[:, None] * dR
    dgam = dgam - b * np.sum(dR * KS, axis=1)
    # KS = K S
    dK = dK + dKS @ S.T
    dS = dS + K.T @ dKS
    # A = b o EA o K K^T (strictly lower)
    dKK = dA * b[:, None] * p["EA"]
    dK = dK + dKK @ K + dKK.T @ K
    db = db + np.sum(dA * p["EA"] * p["KK"], axis=1)
    dD = dA * p["A"]
    # P = EP o Q K^T (lower, with the diagonal)
    dQK = dP * p["EP"]
    dQ = dQ + dQK @ K
    dK = dK + dQK.T @ Q
    dD = dD + dP * p["P"]
    # D = G_r - G_i; gamma = e^G; gamma_C = gamma_{n-1}; w = e^{G_C - G}
    dG = dD.sum(axis=1) - dD.sum(axis=0) + dgam * gam
    dG[n - 1] += dgamC * gam[-1] + np.sum(dw * w)
    dG = dG - dw * w
    # G = cumsum(g)
    dg = np.cumsum(dG[::-1])[::-1]
    return dict(dq=dQ, dk=dK, dv=dV, dg=dg, dbeta=db), dS


def chunked_forward_kda(q, k, v, g, beta, S0=None, cu_seqlens=None, C=64):
    """Chunkwise form with a per-channel log-decay g [ntok, H, dk]. With Gc[r, c] the running
    sum of g over the chunk (per channel), unrolling the recurrence inside a chunk gives
        A[r,i] = beta_r sum_c k_r[c] k_i[c] e^{Gc[r,c] - Gc[i,c]}   (i < r)
        U = (I + A)^{-1} (diag(beta) V - diag(beta) (K o e^{Gc}) S0)
        Y = (Q o e^{Gc}) S0 + P U,   P[r,i] = sum_c q_r[c] k_i[c] e^{Gc[r,c] - Gc[i,c]} (i <= r)
        S_C = Diag(e^{Gc[C]}) S0 + (K o e^{Gc[C] - Gc})^T U"""
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
                Gc = np.cumsum(g[sl, h], axis=0)              # [n, dk]
                b = beta[sl, h]
                n = len(b)
                E = np.exp(np.minimum(Gc[:, None, :] - Gc[None, :, :], 0.0))   # [r, i, c]
                low = np.tril(np.ones((n, n)), -1).astype(bool)
                incl = np.tril(np.ones((n, n))).astype(bool)
                A = np.where(low, b[:, None] * np.einsum("rc,ic,ric->ri", K, K, E), 0.0)
                P = np.where(incl, np.einsum("rc,ic,ric->ri", Q, K, E), 0.0)
                T = np.linalg.inv(np.eye(n) + A)
                U = T @ (b[:, None] * (V - (K * np.exp(Gc)) @ S))
                y[sl, h] = (Q * np.exp(Gc)) @ S + P @ U
                S = np.exp(Gc[-1])[:, None] * S + (K * np.exp(Gc[-1] - Gc)).T @ U
            ST[s, h] = S
    return y, ST
