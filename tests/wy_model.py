"""fp64 numpy model of the chunkwise WY equations the HIP kernels implement.

A debug aid and a check of the chunk equations, not an oracle: test_wy_model.py
compares it with the token-by-token oracle.  Chunk form of the Gated DeltaNet-2
rule (blog on Gated DeltaNet-2, sections on the two-axis control and on the
token path and parallel training):
    Et = (b*k) e^G, Kt = k e^-G, Qt = q e^G, Kh = k e^(g_C - G)
    A = strictly-lower(Et Kt^T), P = lower(Qt Kt^T), T = (I + A)^-1
    U = T (Z - Et S), O = Qt S + P U, S' = diag(e^g_C) S + Kh^T U
and its adjoint per chunk.
"""
import numpy as np


def _chunk_quantities(q, k, v, la, b, w):
    G = np.cumsum(la, axis=0)
    gC = G[-1]
    Et = b * k * np.exp(G)
    Kt = k * np.exp(-G)
    Qt = q * np.exp(G)
    Kh = k * np.exp(gC - G)
    A = np.tril(Et @ Kt.T, -1)
    P = np.tril(Qt @ Kt.T)
    T = np.linalg.inv(np.eye(len(q)) + A)
    return G, gC, Et, Kt, Qt, Kh, A, P, T, w * v


def fwd(q, k, v, la, b, w, S0, C=64):
    """Single (batch, head): token arrays [T, D]; returns (O [T, dv], S_final, start states)."""
    S = S0.copy()
    O = np.zeros((q.shape[0], v.shape[1]))
    starts = []
    for c0 in range(0, q.shape[0], C):
        sl = slice(c0, min(c0 + C, q.shape[0]))
        starts.append(S.copy())
        G, gC, Et, Kt, Qt, Kh, A, P, T, Z = _chunk_quantities(q[sl], k[sl], v[sl], la[sl], b[sl], w[sl])
        U = T @ (Z - Et @ S)
        O[sl] = Qt @ S + P @ U
        S = np.exp(gC)[:, None] * S + Kh.T @ U
    return O, S, starts


def bwd(q, k, v, la, b, w, S0, dO, dSf, C=64):
    """Gradients of sum(dO*O) + sum(dSf*S_final) by the chunk adjoint."""
    _, _, starts = fwd(q, k, v, la, b, w, S0, C)
    out = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dlog_alpha", la), ("db", b),
                                             ("dw", w))}
    dS = dSf.copy()
    chunks = list(range(0, q.shape[0], C))
    for ci in reversed(range(len(chunks))):
        sl = slice(chunks[ci], min(chunks[ci] + C, q.shape[0]))
        S = starts[ci]
        G, gC, Et, Kt, Qt, Kh, A, P, T, Z = _chunk_quantities(q[sl], k[sl], v[sl], la[sl], b[sl], w[sl])
        X = Z - Et @ S
        U = T @ X
        dOc = dO[sl]
        dU = P.T @ dOc + Kh @ dS
        dX = T.T @ dU
        dP = np.tril(dOc @ U.T)
        dA = -np.tril(dX @ U.T, -1)
        dQt = dOc @ S.T + dP @ Kt
        dEt = -dX @ S.T + dA @ Kt
        dKt = dA.T @ Et + dP.T @ Qt
        dKh = U @ dS.T
        dgam = np.sum(dS * S, axis=1)
        gam = np.exp(gC)
        eG, eNG, eK = np.exp(G), np.exp(-G), np.exp(gC - G)
        dE = dEt * eG
        out["dq"][sl] = dQt * eG
        out["db"][sl] = dE * k[sl]
        out["dk"][sl] = dKt * eNG + dKh * eK + dE * b[sl]
        out["dv"][sl] = dX * w[sl]
        out["dw"][sl] = dX * v[sl]
        dG = dQt * Qt + dEt * Et - dKt * Kt - dKh * Kh
        dgC = np.sum(dKh * Kh, axis=0) + dgam * gam
        out["dlog_alpha"][sl] = np.cumsum(dG[::-1], axis=0)[::-1] + dgC
        dS = Qt.T @ dOc + gam[:, None] * dS - Et.T @ dX
    out["dS0"] = dS
    return out
