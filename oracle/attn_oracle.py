"""FP64 oracle of packed-varlen causal GQA training attention (head dim 256).

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and the ``cpu_baseline`` leg
of ``bench.py``. The product library never imports, links or runs anything in
this directory.

What it computes (flashinfer PR #7774, description and commit notes: dense
GQA attention over inputs packed by cu_seqlens, a causal mask aligned to the
bottom right of each segment so that query and key lengths may differ, the
forward with the natural-log LSE, and a backward whose dK / dV are sums over
the query heads that share each key head). Per segment s with queries
[cq_s, cq_s+1) (Lq of them) and keys [ck_s, ck_s+1) (Lk), query head h and its
key head g = h // (Hq / Hkv):

    S[i, j]  = scale * <q_i, k_j>               for j <= i + (Lk - Lq), else masked
    lse_i    = log sum_j exp(S[i, j])           (-inf for a row that sees no key)
    P[i, j]  = exp(S[i, j] - lse_i)
    o_i      = sum_j P[i, j] v_j                (0 for a row that sees no key)

and the backward of L = sum <o, dO>:

    dP = dO V^T,  Delta_i = <dO_i, o_i>,  dS = P * (dP - Delta)
    dq = scale dS K,  dk_g = scale sum_{h in g} dS^T Q_h,  dv_g = sum_{h in g} P^T dO_h

Every array is float64; the loops run over segments and heads, each step a
plain matrix expression.
"""

from __future__ import annotations

import numpy as np


def _segments(cu_q, cu_k):
    cu_q = np.asarray(cu_q, np.int64)
    cu_k = np.asarray(cu_k, np.int64)
    return [(int(cu_q[s]), int(cu_q[s + 1]), int(cu_k[s]), int(cu_k[s + 1]))
            for s in range(len(cu_q) - 1)]


def _mask(Lq, Lk):
    """True where query i (0-based in the segment) may see key j."""
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    return j <= i + (Lk - Lq)


def attn_fwd(cu_q, cu_k, q, k, v, scale=None):
    """o [Tq, Hq, D] and lse [Tq, Hq] (float64)."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    grp = Hq // Hkv
    scale = D ** -0.5 if scale is None else scale
    o = np.zeros((Tq, Hq, D))
    lse = np.full((Tq, Hq), -np.inf)
    for a, b, c, e in _segments(cu_q, cu_k):
        Lq, Lk = b - a, e - c
        if Lq == 0:
            continue
        m = _mask(Lq, Lk)
        for h in range(Hq):
            g = h // grp
            S = scale * q[a:b, h] @ k[c:e, g].T
            S = np.where(m, S, -np.inf)
            mx = np.max(S, axis=1, keepdims=True) if Lk else np.full((Lq, 1), -np.inf)
            seen = np.isfinite(mx[:, 0])
            if not seen.any():
                continue
            ex = np.exp(S[seen] - mx[seen])
            den = ex.sum(axis=1, keepdims=True)
            lse[a:b, h][seen] = (mx[seen] + np.log(den))[:, 0]
            o[a:b, h][seen] = (ex / den) @ v[c:e, g]
    return o, lse


def attn_bwd(cu_q, cu_k, q, k, v, dO, scale=None):
    """Gradients of L = sum(o * dO): dict with dq [Tq, Hq, D], dk and dv
    [Tk, Hkv, D] (float64), each dk / dv the sum over its query heads."""
    q, k, v, dO = (np.asarray(a, np.float64) for a in (q, k, v, dO))
    Tq, Hq, D = q.shape
    Tk, Hkv = k.shape[:2]
    grp = Hq // Hkv
    scale = D ** -0.5 if scale is None else scale
    o, lse = attn_fwd(cu_q, cu_k, q, k, v, scale)
    dq = np.zeros_like(q)
    dk = np.zeros((Tk, Hkv, D))
    dv = np.zeros((Tk, Hkv, D))
    for a, b, c, e in _segments(cu_q, cu_k):
        Lq, Lk = b - a, e - c
        if Lq == 0 or Lk == 0:
            continue
        m = _mask(Lq, Lk)
        for h in range(Hq):
            g = h // grp
            fin = np.isfinite(lse[a:b, h])[:, None]      # rows that see a key
            L = np.where(fin, lse[a:b, h][:, None], 0.0)
            S = scale * q[a:b, h] @ k[c:e, g].T
            P = np.where(m & fin, np.exp(np.where(m, S, -np.inf) - L), 0.0)
            dP = dO[a:b, h] @ v[c:e, g].T
            delta = np.sum(dO[a:b, h] * o[a:b, h], axis=1, keepdims=True)
            dS = P * (dP - delta)
            dq[a:b, h] = scale * dS @ k[c:e, g]
            dk[c:e, g] += scale * dS.T @ q[a:b, h]
            dv[c:e, g] += P.T @ dO[a:b, h]
    return {"dq": dq, "dk": dk, "dv": dv}
