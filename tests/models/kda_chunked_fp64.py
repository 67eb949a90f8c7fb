"""FP64 chunked form of the gated delta rule (test-only model).

A second, independent formulation of what the oracle computes: the chunked
training form (per-chunk gate cumsum, UT/WY triangular solve, intra-chunk
products, inter-chunk affine state map S_out = M S_in + B; flashinfer PR #7176
opening section describes the per-chunk FP32 affine state summary, PR #8909
opening section the chunked training package). In exact arithmetic it equals
the token-by-token recurrence, so agreement between the two to ~1e-12 pins
both. It works on already-transformed inputs (gate g, L2 norm applied).

Per chunk of n tokens inside one document, with G the inclusive cumsum of g:
  Kd = K*e^G, Qd = Q*e^G, Ke = K*e^(G_last - G), gam = e^(G_last)
  A_kk[r,i] = sum_c k_r k_i e^(G_r - G_i)  (i < r),  A_qk likewise (i <= r)
  T = (I + diag(beta) A_kk)^-1,  Tb = T diag(beta)
  R = V - Kd S,  U~ = Tb R,  O = scale (Qd S + A_qk U~),  S' = gam*S + Ke^T U~
and the reverse pass of the same steps.
"""

from __future__ import annotations

import numpy as np


def _chunk_terms(q, k, g, beta):
    n = q.shape[0]
    G = np.cumsum(g, axis=0)
    mask_lt = np.tril(np.ones((n, n)), -1)
    mask_le = np.tril(np.ones((n, n)), 0)
    diff = np.where(mask_le[:, :, None] > 0, G[:, None, :] - G[None, :, :], -np.inf)
    E = np.exp(diff)                                      # [r, i, c], 0 above the diagonal
    Akk = np.einsum("rc,ic,ric->ri", k, k, E) * mask_lt
    Aqk = np.einsum("rc,ic,ric->ri", q, k, E) * mask_le
    T = np.linalg.inv(np.eye(n) + beta[:, None] * Akk)
    T = np.tril(T)
    return G, E, Akk, Aqk, T, mask_lt, mask_le


def forward(cu, q, k, v, beta, g, scale, C=64):
    """o [T,H,V] and the state at every chunk start [n_chunks,H,K,V]."""
    T_, H, K = q.shape
    V = v.shape[2]
    o = np.zeros((T_, H, V))
    starts = []
    for d in range(len(cu) - 1):
        for s in range(cu[d], cu[d + 1], C):
            starts.append((d, s, min(s + C, cu[d + 1])))
    S_in = np.zeros((len(starts), H, K, V))
    for h in range(H):
        S = None
        for ci, (d, s, e) in enumerate(starts):
            if s == cu[d]:
                S = np.zeros((K, V))
            S_in[ci, h] = S
            qc, kc, vc, bc, gc = q[s:e, h], k[s:e, h], v[s:e, h], beta[s:e, h], g[s:e, h]
            G, E, Akk, Aqk, Tm, _, _ = _chunk_terms(qc, kc, gc, bc)
            Kd, Qd = kc * np.exp(G), qc * np.exp(G)
            Ke = kc * np.exp(G[-1] - G)
            Tb = Tm * bc[None, :]
            R = vc - Kd @ S
            U = Tb @ R
            o[s:e, h] = scale * (Qd @ S + Aqk @ U)
            S = np.exp(G[-1])[:, None] * S + Ke.T @ U
    return o, S_in


def backward(cu, q, k, v, beta, g, dO, scale, C=64):
    """Gradients of L = sum(o*dO) w.r.t. q, k, v, beta, g (already transformed)."""
    T_, H, K = q.shape
    V = v.shape[2]
    _, S_all = forward(cu, q, k, v, beta, g, scale, C)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dbeta, dg = np.zeros_like(beta), np.zeros_like(g)
    starts = []
    for d in range(len(cu) - 1):
        for s in range(cu[d], cu[d + 1], C):
            starts.append((d, s, min(s + C, cu[d + 1])))
    for h in range(H):
        dS = None
        for ci in range(len(starts) - 1, -1, -1):
            d, s, e = starts[ci]
            if e == cu[d + 1]:
                dS = np.zeros((K, V))
            S = S_all[ci, h]
            qc, kc, vc, bc, gc = q[s:e, h], k[s:e, h], v[s:e, h], beta[s:e, h], g[s:e, h]
            dOc = dO[s:e, h]
            G, E, Akk, Aqk, Tm, mlt, mle = _chunk_terms(qc, kc, gc, bc)
            eG = np.exp(G)
            Kd, Qd = kc * eG, qc * eG
            eL = np.exp(G[-1] - G)
            Ke = kc * eL
            gam = np.exp(G[-1])
            Tb = Tm * bc[None, :]
            R = vc - Kd @ S
            U = Tb @ R
            # state-passing part
            dU = scale * Aqk.T @ dOc + Ke @ dS
            dR = Tb.T @ dU
            dS_in = gam[:, None] * dS + scale * Qd.T @ dOc - Kd.T @ dR
            dQd = scale * dOc @ S.T
            dKd = -dR @ S.T
            dKe = U @ dS.T
            dgam = np.sum(dS * S, axis=1)
            dAqk = scale * (dOc @ U.T) * mle
            dTb = (dU @ R.T) * mle
            # WY / UT solve
            dT = dTb * bc[None, :]
            db = np.sum(dTb * Tm, axis=0)
            dX = -(Tm.T @ dT @ Tm.T) * mlt
            dAkk = bc[:, None] * dX
            db += np.sum(dX * Akk, axis=1)
            dvc = dR
            # intra products through q, k, G
            dqc = dQd * eG + np.einsum("ri,ic,ric->rc", dAqk, kc, E)
            dkc = (dKd * eG + dKe * eL
                   + np.einsum("ri,rc,ric->ic", dAqk, qc, E)
                   + np.einsum("ri,ic,ric->rc", dAkk, kc, E)
                   + np.einsum("ri,rc,ric->ic", dAkk, kc, E))
            P_qk = np.einsum("ri,rc,ic,ric->ric", dAqk, qc, kc, E)
            P_kk = np.einsum("ri,rc,ic,ric->ric", dAkk, kc, kc, E)
            P = P_qk + P_kk
            dG = dKd * Kd + dQd * Qd - dKe * Ke + P.sum(axis=1) - P.sum(axis=0)
            dG[-1] += np.sum(dKe * Ke, axis=0) + dgam * gam
            dgc = np.cumsum(dG[::-1], axis=0)[::-1]
            dq[s:e, h], dk[s:e, h], dv[s:e, h] = dqc, dkc, dvc
            dbeta[s:e, h], dg[s:e, h] = db, dgc
            dS = dS_in
    return {"dq": dq, "dk": dk, "dv": dv, "dbeta": dbeta, "dg": dg}
