"""The gated delta rule's backward in its chunkwise form agrees with the oracle's.

The oracle's ``gdelta_backward`` is reverse mode through the recurrent form (the
gates page, section "Unire oblio e correzione: Gated DeltaNet"). The GPU path
differentiates the chunkwise UT form instead (section "Correggere: la delta rule";
RetNet page, Fig. 16.5): per chunk, the pseudo-values U = T diag(beta) (V - diag(e^G)
K S^T), the memory's gradient carried back chunk by chunk, and each chunk's input
gradients from the records. Here those chunk formulas are written out in float64
numpy (no code shared with the kernels or the oracle) and must reproduce the
oracle's gradients of every input to rounding, across chunk lengths, a ragged tail,
an initial memory and a gradient of the final memory: a second, independent pin of
the oracle's backward.
"""

import numpy as np
import pytest

import oracle as orc


def _chunk_backward(Q, K, V, LA, BE, DO, S0, DST, C):
    """One sequence: (dq, dk, dv, dlog_alpha, dbeta, ds0) by the chunkwise reverse mode."""
    T = Q.shape[0]
    NC = (T + C - 1) // C
    S = S0.copy()
    recs = []
    for c in range(NC):
        sl = slice(c * C, min(T, c * C + C))
        q_, k_, v_, a_, b_ = Q[sl], K[sl], V[sl], LA[sl], BE[sl]
        n = len(a_)
        G = np.cumsum(a_)
        g, w = np.exp(G), np.exp(G[-1] - G)
        Gam = np.exp(G[:, None] - G[None, :])
        KK = k_ @ k_.T
        A = np.tril(b_[:, None] * KK * Gam, -1)
        Tm = np.linalg.inv(np.eye(n) + A)
        TU = Tm * b_[None, :]
        R = v_ - g[:, None] * (k_ @ S.T)
        U = TU @ R
        P = np.tril((q_ @ k_.T) * Gam)
        recs.append((sl, S.copy(), U, R, P, Tm, TU, g, w, Gam, KK, G))
        S = np.exp(G[-1]) * S + U.T @ (w[:, None] * k_)
    dS = DST.copy()
    out = [np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V), np.zeros_like(LA), np.zeros_like(BE)]
    for sl, Sin, U, R, P, Tm, TU, g, w, Gam, KK, G in reversed(recs):
        q_, k_, b_, dO = Q[sl], K[sl], BE[sl], DO[sl]
        n = len(g)
        low = np.tril(np.ones((n, n)), -1)
        dU = P.T @ dO + w[:, None] * (k_ @ dS.T)
        dR = TU.T @ dU
        dP = (dO @ U.T) * np.tril(np.ones((n, n)))
        dPG = dP * Gam
        dTU = dU @ R.T
        dA = np.tril(-Tm.T @ (dTU * b_[None, :]) @ Tm.T, -1)
        M = dA * b_[:, None] * Gam
        Z2, Z = dR @ Sin, U @ dS
        out[0][sl] = g[:, None] * (dO @ Sin) + dPG @ k_
        out[1][sl] = dPG.T @ q_ + (M + M.T) @ k_ - g[:, None] * Z2 + w[:, None] * Z
        out[2][sl] = dR
        out[4][sl] = (dTU * Tm).sum(0) + (dA * KK * Gam).sum(1)
        Am = b_[:, None] * KK * Gam * low
        dw = (Z * k_).sum(1)
        dG = (g * ((dO @ Sin) * q_).sum(1) - g * (Z2 * k_).sum(1) + (dP * P).sum(1) - (dP * P).sum(0)
              + (dA * Am).sum(1) - (dA * Am).sum(0) - w * dw)
        dG[-1] += (w * dw).sum() + np.exp(G[-1]) * (dS * Sin).sum()
        out[3][sl] = np.cumsum(dG[::-1])[::-1]
        dS = np.exp(G[-1]) * dS + dO.T @ (g[:, None] * q_) - dR.T @ (g[:, None] * k_)
    return out + [dS]


@pytest.mark.parametrize("T,dk,dv,C", [(150, 16, 12, 64), (37, 8, 5, 16), (64, 6, 9, 32), (1, 4, 4, 64)])
def test_chunkwise_reverse_mode_matches_oracle(T, dk, dv, C):
    rng = np.random.default_rng(T + 7 * dk + C)
    q = rng.standard_normal((1, 1, T, dk)) * 0.5
    k = rng.standard_normal((1, 1, T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, 1, T, dv))
    la = -np.abs(rng.standard_normal((1, 1, T))) * 0.3
    be = 1.0 / (1.0 + np.exp(-rng.standard_normal((1, 1, T))))
    do = rng.standard_normal((1, 1, T, dv))
    dST = rng.standard_normal((1, 1, dv, dk)) * 0.1
    s0 = rng.standard_normal((1, 1, dv, dk)) * 0.1
    ref = orc.gdelta_backward(q, k, v, la, be, do, dS_T=dST, s0=s0)
    got = _chunk_backward(q[0, 0], k[0, 0], v[0, 0], la[0, 0], be[0, 0], do[0, 0], s0[0, 0], dST[0, 0], C)
    for name, a, r in zip(("dq", "dk", "dv", "dlog_alpha", "dbeta", "ds0"), got, ref):
        r = np.asarray(r, dtype=np.float64)[0, 0]
        assert np.abs(a - r).max() <= 1e-12 * max(np.abs(r).max(), 1.0), name
