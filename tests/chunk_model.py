"""fp64 numpy model of the chunkwise (UT/WY) form of the KDA recurrence.

A second, independent derivation used only to pin the oracle and to lock the
algebra the GPU prefill kernel follows.  The pages state the chunk interface
(X_[c], S_in) -> (Y_[c], S_out) with S_in of chunk c+1 equal to S_out of chunk
c, name the WY/UT organisation and the 16-position secondary tile, but print no
derivation (page "Kimi K3：架构、训练与百万 Token Agentic RL 技术解读", section
3.3).  The derivation used here: inside a chunk with incoming state S and
chunk-relative cumulative log-decay G_r = sum_{s<=r} g_s,
    A[r,i] = beta_r sum_c k[r,c] k[i,c] exp(G[r,c] - G[i,c])      (i < r)
    M[r,i] =        sum_c q[r,c] k[i,c] exp(G[r,c] - G[i,c])      (i <= r)
    U      = (I + A)^{-1} Diag(beta) (V - (k*exp(G)) S)
    O      = (q*exp(G)) S + M U
    S_out  = Diag(exp(G_C)) S + (k*exp(G_C - G))^T U
`ref` selects where each exp(G_r - G_i) is split into a row and a column factor:
    "direct"  -- the product is formed from the difference (no split),
    "center"  -- split at the middle of the chunk (each factor then spans at most
                 C/2 positions of decay),
    "start"   -- split at the chunk start, as the chunk-16 GPU kernel does (row
                 factor exp(G_r) <= 1, column factor exp(-G_i) <= e^{5 C}).
`inverse` selects how (I + A)^{-1} is formed:
    "solve"   -- a dense linear solve,
    "product" -- the exact finite product (I - A)(I + A^2)(I + A^4)(I + A^8) for a
                 strictly lower triangular A of order <= 16 (A^16 = 0), as the
                 chunk-16 GPU kernel evaluates it.
"""
import numpy as np


def nilpotent_inverse(A):
    """(I + A)^{-1} for strictly lower triangular A of order n <= 16, as the product
    (I - A)(I + A^2)(I + A^4)(I + A^8) = sum_{j<16} (-A)^j (A^16 = 0)."""
    n = A.shape[0]
    assert n <= 16 and not np.triu(A).any()
    I = np.eye(n)
    A2 = A @ A
    A4 = A2 @ A2
    A8 = A4 @ A4
    return (I - A) @ (I + A2) @ (I + A4) @ (I + A8)


def chunk_forward(q, k, v, g, beta, S0, C, ref="direct", inverse="solve", dtype=np.float64):
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv), dtype=dtype) if S0 is None else np.array(S0, dtype=dtype)
    o = np.zeros((T, dv), dtype=dtype)
    for c0 in range(0, T, C):
        sl = slice(c0, min(T, c0 + C))
        qc, kc, vc, gc, bc = q[sl], k[sl], v[sl], g[sl], beta[sl]
        n = qc.shape[0]
        G = np.cumsum(gc, axis=0)
        if ref == "direct":
            D = G[:, None, :] - G[None, :, :]                    # [r, i, c]
            E = np.exp(np.where(np.arange(n)[:, None, None] >= np.arange(n)[None, :, None], D, -np.inf))
            KK = np.einsum("rc,ic,ric->ri", kc, kc, E)
            QK = np.einsum("rc,ic,ric->ri", qc, kc, E)
        elif ref == "start":
            rowf = np.exp(G)
            colf = np.exp(-G)
            KK = (kc * rowf) @ (kc * colf).T
            QK = (qc * rowf) @ (kc * colf).T
        elif ref == "center":
            h = min(C // 2, n)
            R = G[h - 1]
            rowf = np.exp(G - R)
            colf = np.exp(R - G)
            KK = (kc * rowf) @ (kc * colf).T
            QK = (qc * rowf) @ (kc * colf).T
        else:
            raise ValueError(ref)
        A = np.tril(bc[:, None] * KK, -1)
        M = np.tril(QK)
        if inverse == "solve":
            Tm = np.linalg.solve(np.eye(n, dtype=A.dtype) + A, np.diag(bc))
        elif inverse == "product":
            Tm = nilpotent_inverse(A) @ np.diag(bc)
        else:
            raise ValueError(inverse)
        U = Tm @ (vc - (kc * np.exp(G)) @ S)
        o[sl] = (qc * np.exp(G)) @ S + M @ U
        S = np.exp(G[-1])[:, None] * S + (kc * np.exp(G[-1] - G)).T @ U
    return o, S


def chunk_backward(q, k, v, g, beta, S0, dO, dS_T, C, inverse="solve", dtype=np.float64,
                   flush_subnormal=False):
    """Gradients of <dO, o> + <dS_T, S_T> through the chunk form above (one head),
    by reverse-mode differentiation of each chunk's matrix expressions, chunks in
    reverse order with the incoming state of each chunk from a forward pass.
    With chunk-relative G (cumulative log-decay), P = exp(G), Gam = P[-1]:
        Kt = k P, Qt = q P, Kc = k / P, Ke = k Gam / P,  B = Kt Kc^T,
        A = strict_lower(Diag(beta) B), L = (I + A)^{-1}, Tm = L Diag(beta),
        X = V - Kt S, U = Tm X, M = lower(Qt Kc^T),
        O = Qt S + M U,  S' = Diag(Gam) S + Ke^T U.
    Returns (dq, dk, dv, dg, dbeta, dS0) as arrays of `dtype` (float64 by default; with
    float32 every step rounds to float32).  flush_subnormal sets the Kt entries below the
    smallest normal number of `dtype` to zero, as matrix units that flush sub-normal
    operands see them."""
    q, k, v, g, beta, dO = (np.asarray(x, dtype=dtype) for x in (q, k, v, g, beta, dO))
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv), dtype=dtype) if S0 is None else np.array(S0, dtype=dtype)
    starts = []                                   # incoming state of every chunk
    for c0 in range(0, T, C):
        starts.append(S.copy())
        sl = slice(c0, min(T, c0 + C))
        _, S = chunk_forward(q[sl], k[sl], v[sl], g[sl], beta[sl], S, C, ref="direct", inverse=inverse,
                             dtype=dtype)
    dq, dk_, dv_, dg, db = (np.zeros_like(x) for x in (q, k, v, g, beta))
    dSn = np.array(dS_T, dtype=dtype)             # gradient w.r.t. the chunk's outgoing state
    for ci in range(len(starts) - 1, -1, -1):
        c0 = ci * C
        sl = slice(c0, min(T, c0 + C))
        qc, kc, vc, gc, bc, dOc = q[sl], k[sl], v[sl], g[sl], beta[sl], dO[sl]
        S = starts[ci]
        n = qc.shape[0]
        G = np.cumsum(gc, axis=0)
        P = np.exp(G)
        Gam = P[-1]
        Kt, Qt, Kc, Ke = kc * P, qc * P, kc / P, kc * (Gam / P)
        if flush_subnormal:
            tiny = np.finfo(dtype).tiny
            Kt = np.where(np.abs(Kt) < tiny, 0, Kt).astype(dtype)
        B = Kt @ Kc.T
        A = np.tril(bc[:, None] * B, -1)
        I = np.eye(n, dtype=dtype)
        L = np.linalg.solve(I + A, I) if inverse == "solve" else nilpotent_inverse(A)
        Tm = L * bc[None, :]
        X = vc - Kt @ S
        U = Tm @ X
        M = np.tril(Qt @ Kc.T)
        # reverse mode
        dU = M.T @ dOc + Ke @ dSn
        dM = np.tril(dOc @ U.T)
        dQt = dOc @ S.T + dM @ Kc
        dKc = dM.T @ Qt
        dKe = U @ dSn.T
        dX = Tm.T @ dU
        dTm = dU @ X.T
        dKt = -dX @ S.T
        dS = Qt.T @ dOc + Gam[:, None] * dSn - Kt.T @ dX
        dL = dTm * bc[None, :]
        dbc = np.sum(L * dTm, axis=0)
        dA = np.tril(-L.T @ dL @ L.T, -1)
        dbc += np.sum(dA * B, axis=1)
        dB = bc[:, None] * dA
        dKt += dB @ Kc
        dKc += dB.T @ Kt
        dk_[sl] = dKt * P + dKc / P + dKe * (Gam / P)
        dq[sl] = dQt * P
        dG = dKt * Kt + dQt * Qt - dKc * Kc - dKe * Ke
        dG[-1] += np.sum(dSn * S, axis=1) * Gam + np.sum(dKe * Ke, axis=0)
        dg[sl] = np.cumsum(dG[::-1], axis=0)[::-1]
        dv_[sl] = dX
        db[sl] = dbc
        dSn = dS
    return dq, dk_, dv_, dg, db, dSn
