"""FP64 oracle of the width-4 causal conv1d + SiLU training op over packed
documents, with a halo.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and the ``cpu_baseline`` leg
of ``bench.py``. The product library never imports, links or runs anything in
this directory.

What it computes. The KDA module forward runs a width-4 causal conv1d + SiLU
in front of the state passing, and the context-parallel route ships a halo
variant of that conv so that a document split across fragments sees the tokens
before its fragment (flashinfer PR #7176, measurement paragraph of the
description: module forward = conv halo + conv + state passing; and the
paragraph on the family's other variants: the halo variant of the width-4
causal conv1d + SiLU training backend). The pages print no formula; the plain
reading, per channel c of a packed [T, D] input x with document starts s_d:

    z[t, c] = b[c] + sum_{j=0..W-1} w[c, j] * xx(t - (W-1) + j, c)
    y[t, c] = z[t, c] * sigmoid(z[t, c])                       (SiLU)

    xx(u, c) = x[u, c]                   if u >= s(t), the start of t's document
             = halo[(W-1) + (u - s_0), c] if t is in document 0 and a halo is given
                                          (the W-1 tokens right before x[0], oldest first)
             = 0                          otherwise (a document start sees zeros)

so w[c, W-1] multiplies the current token and w[c, 0] the oldest. The backward
of L = sum(y * dy) is written out by hand from these two lines:

    dz = dy * (s + z s (1 - s)),  s = sigmoid(z)
    dx[u, c]    = sum_j w[c, j] dz[u + (W-1) - j, c]   over tokens of u's document
    dw[c, j]    = sum_t dz[t, c] xx(t - (W-1) + j, c)
    db[c]       = sum_t dz[t, c]
    dhalo[i, c] = sum_j w[c, j] dz[i - j, c]            over t = i - j in [0, len_0)

Every array is float64; loops run over the W taps and the documents, with each
step vectorised over tokens and channels.
"""

from __future__ import annotations

import numpy as np

WIDTH = 4


def _sigmoid(z):
    e = np.exp(-np.abs(z))          # never overflows
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def _shifted(x, cu, shift, halo=None):
    """xx(t - shift, c) for every t: x shifted down by `shift` tokens inside
    each document, zeros before a document start, the halo before document 0."""
    T, D = x.shape
    out = np.zeros((T, D))
    for d in range(len(cu) - 1):
        a, e = int(cu[d]), int(cu[d + 1])
        if e - a > shift:
            out[a + shift:e] = x[a:e - shift]
        if d == 0 and halo is not None:
            # tokens t = a .. a + shift - 1 reach back before the document start
            for t in range(a, min(e, a + shift)):
                out[t] = halo[(WIDTH - 1) + (t - a) - shift]
    return out


def conv_silu_fwd(cu, x, w, b=None, halo=None):
    """y [T, D] and the pre-activation z [T, D] (float64)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    T, D = x.shape
    z = np.zeros((T, D)) if b is None else np.broadcast_to(np.asarray(b, np.float64), (T, D)).copy()
    for j in range(WIDTH):
        z += w[:, j][None, :] * _shifted(x, cu, (WIDTH - 1) - j, halo)
    return z * _sigmoid(z), z


def conv_silu_bwd(cu, x, w, dy, b=None, halo=None):
    """Gradients of L = sum(y * dy): dict with dx [T, D], dw [D, W], db [D]
    and, with a halo, dhalo [W-1, D] (float64)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    dy = np.asarray(dy, np.float64)
    T, D = x.shape
    _, z = conv_silu_fwd(cu, x, w, b, halo)
    s = _sigmoid(z)
    dz = dy * (s + z * s * (1.0 - s))
    dx = np.zeros((T, D))
    dw = np.zeros((D, WIDTH))
    for j in range(WIDTH):
        shift = (WIDTH - 1) - j
        dw[:, j] = np.sum(dz * _shifted(x, cu, shift, halo), axis=0)
        # x[u] feeds z[u + shift] through tap j, inside u's document
        for d in range(len(cu) - 1):
            a, e = int(cu[d]), int(cu[d + 1])
            if e - a > shift:
                dx[a:e - shift] += w[:, j][None, :] * dz[a + shift:e]
    out = {"dx": dx, "dw": dw, "db": np.sum(dz, axis=0)}
    if halo is not None:
        dhalo = np.zeros((WIDTH - 1, D))
        a, e = int(cu[0]), int(cu[1])
        for i in range(WIDTH - 1):
            for j in range(WIDTH):
                t = a + i - j          # halo row i is token a - (W-1) + i, seen by z[t] through tap j
                if a <= t < e:
                    dhalo[i] += w[:, j] * dz[t]
        out["dhalo"] = dhalo
    return out
