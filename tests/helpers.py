"""Shared helpers for the tests: random tiny problems and error metrics."""

import numpy as np


def rel_l2(x, ref):
    """||x - ref||_2 / ||ref||_2 in float64 over the whole tensor."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    if den == 0.0:
        return float(num)
    return float(num / den)


def tiny_problem(rng, doc_lens, H, K, V, gate="g", l2norm=False, decay=0.3, alog_hi=1.4):
    """Random FP64 inputs of arbitrary (small) sizes for oracle pins."""
    T = int(sum(doc_lens))
    cu = np.concatenate([[0], np.cumsum(doc_lens)]).astype(np.int64)
    q = rng.standard_normal((T, H, K))
    k = rng.standard_normal((T, H, K))
    if not l2norm:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, V))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    p = dict(cu=cu, q=q, k=k, v=v, beta=beta, dO=rng.standard_normal((T, H, V)),
             gate_form=gate, l2norm=l2norm)
    if gate == "g":
        p["gate"] = -decay * np.abs(rng.standard_normal((T, H, K)))
    else:
        p["gate"] = rng.standard_normal((T, H, K))
        p["A_log"] = rng.uniform(0.0, alog_hi, H)
        p["dt_bias"] = rng.normal(0.0, 0.5, (H, K))
    return p
