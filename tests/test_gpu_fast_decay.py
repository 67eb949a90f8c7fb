"""Parity under very fast decay, where the decayed products of a chunk span
hundreds of nats: per-step decays of e^-15 .. e^-1200 (A_log up to ln 256)
make every diagonal 16-row block too wide for a shared reference, so the
running-product sums of the forward prep and of the per-chunk backward carry
the diagonal blocks, and most factors underflow to zero. A third case puts
block spans around the calm limits (40 in the backward, 120 in the prep).

The gated delta rule and its chunked form are those of flashinfer PR #8909
(opening section) with packed documents as in PR #7176 (opening section); the
oracle is the FP64 token recurrence, on the same seeded inputs.

dA_log[h] = sum_{t,c} dg g and ddt_bias[h,c] = sum_t da are sums whose terms
cancel by factors of 10^2 .. 10^3 under fast decay (measured on the oracle).
They keep the whole-vector relative-L2 bound of every gate gradient (1e-2);
the error relative to the sum of the terms' magnitudes (sum |dg g| per head,
sum |da| per head and channel, from the oracle) is printed beside it.
"""

import numpy as np
import pytest

from gpu_common import TOL, f64, gpu_grads_f64, rel_l2, run_gpu, run_oracle, to_device
from kda_chunked_amd import inputs as I

pytestmark = pytest.mark.gpu

CASES = [
    ("extreme", (float(np.log(64.0)), float(np.log(256.0))), [200, 77, 300], False),
    ("steep", (float(np.log(16.0)), float(np.log(64.0))), [200, 77, 300], False),
    ("near-calm", (float(np.log(2.0)), float(np.log(8.0))), [257, 130], True),
]


def _term_scales(inp, gref):
    """Sum of |dg g| per head and of |da| per (head, channel), from the oracle."""
    f = I.as_f64(inp)
    ea = np.exp(f["A_log"])[None, :, None]
    z = f["gate"] + f["dt_bias"][None]
    g = -ea * np.logaddexp(0.0, z)
    sig = 1.0 / (1.0 + np.exp(-z))
    dg = gref["da"] / (-ea * sig)
    return np.abs(dg * g).sum(axis=(0, 2)), np.abs(gref["da"]).sum(axis=0)


@pytest.mark.parametrize("name,alog,docs,l2", CASES, ids=[c[0] for c in CASES])
def test_fast_decay_parity(name, alog, docs, l2):
    w = I.custom(docs, 2, gate="raw", l2norm=l2, alog_range=alog, seed=31, name=name)
    print(f"[case] fast decay {w.key} docs={w.doc_lens} A_log in {alog}", flush=True)
    inp = I.make_inputs(w)
    dev = to_device(inp)
    o, g, _ = run_gpu(w, dev)
    oref, gref = run_oracle(w, inp)
    gg = gpu_grads_f64(w, g)
    errs = {"o": rel_l2(f64(o), oref)}
    errs.update({k: rel_l2(gg[k], v) for k, v in gref.items() if k not in ("dA_log", "ddt_bias")})
    sA, sdt = _term_scales(inp, gref)
    errs["dA_log/sum|terms|"] = float(np.max(np.abs(gg["dA_log"] - gref["dA_log"]) / sA))
    errs["ddt_bias/sum|terms|"] = float(np.max(np.abs(gg["ddt_bias"] - gref["ddt_bias"]) / sdt))
    errs["dA_log"] = rel_l2(gg["dA_log"], gref["dA_log"])
    errs["ddt_bias"] = rel_l2(gg["ddt_bias"], gref["ddt_bias"])
    print(f"[parity] {name} " + ", ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if k in TOL and not v <= TOL[k]}
    assert not bad, bad
