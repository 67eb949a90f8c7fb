"""GPU properties beyond parity: bitwise determinism, saved == replay,
document isolation, ragged and empty documents, many short documents, and
outputs that never depend on the prior contents of the output, saved-set or
workspace buffers (every region the library reads is one it wrote first).

The bitwise properties are stated by the deterministic KDA package (flashinfer
PR #8909, opening section: bitwise reproducible forward and backward); the
ragged cases follow the packed-document layout of flashinfer PR #7176 (opening
section). Values are compared with the FP64 oracle where a tolerance applies.
"""

import numpy as np
import pytest
import torch

from gpu_common import TOL, f64, gpu_grads_f64, rel_l2, run_gpu, run_oracle, to_device
from kda_chunked_amd import inputs as I
from kda_chunked_amd.binding import KDA

pytestmark = pytest.mark.gpu

GRAD_KEYS = ("dq", "dk", "dv", "dbeta", "dgate", "dA_log", "ddt_bias")


def _same_bits(a, b):
    return a.shape == b.shape and a.dtype == b.dtype and torch.equal(
        a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _outputs(o, g):
    out = {"o": o}
    out.update({k: g[k] for k in GRAD_KEYS if k in g and g[k] is not None})
    return out


@pytest.mark.parametrize("name", ["R2", "1doc", "4doc"])
def test_bitwise_deterministic(name):
    w = I.BY_NAME[name]
    print(f"[case] determinism {w.key}", flush=True)
    dev = to_device(I.make_inputs(w))
    o1, g1, _ = run_gpu(w, dev)
    first = {k: v.clone() for k, v in _outputs(o1, g1).items()}
    del o1, g1
    o2, g2, _ = run_gpu(w, dev)          # fresh buffers and workspace
    for k, v in _outputs(o2, g2).items():
        assert _same_bits(first[k], v), f"{w.key}: {k} differs between runs"


@pytest.mark.parametrize("name", ["R2", "4doc"])
def test_replay_is_bitwise_saved(name):
    w = I.BY_NAME[name]
    print(f"[case] replay == saved {w.key}", flush=True)
    dev = to_device(I.make_inputs(w))
    _, gs, _ = run_gpu(w, dev, replay=False)
    saved = {k: v.clone() for k, v in gs.items() if v is not None}
    del gs
    _, gr, _ = run_gpu(w, dev, replay=True)
    for k, v in saved.items():
        assert _same_bits(v, gr[k]), f"{w.key}: {k} differs between saved and replay"


def _poison_run(w, dev, fill):
    """Forward + backward with every output, the saved set and the workspace
    pre-filled with the byte `fill`."""
    kda = KDA(w.T, w.H, len(w.doc_lens), gate=w.gate, l2norm=w.l2norm)
    kda.saved.fill_(fill)
    kda.workspace.fill_(fill)
    o = torch.empty_like(dev["v"])
    o.view(torch.uint8).fill_(fill)
    out = dict(dq=torch.empty_like(dev["q"]), dk=torch.empty_like(dev["k"]),
               dv=torch.empty_like(dev["v"]), dbeta=torch.empty_like(dev["beta"]),
               dgate=torch.empty_like(dev["gate"]))
    if w.gate == "raw":
        out.update(dA_log=torch.empty_like(dev["A_log"]), ddt_bias=torch.empty_like(dev["dt_bias"]))
    for t in out.values():
        t.view(torch.uint8).fill_(fill)
    args = (dev["q"], dev["k"], dev["v"], dev["beta"], dev["gate"], dev["cu_seqlens"])
    kda.forward(*args, dev.get("A_log"), dev.get("dt_bias"), save=True, o=o)
    kda.backward(*args, dev["dO"], dev.get("A_log"), dev.get("dt_bias"), out=out)
    torch.cuda.synchronize()
    return _outputs(o, out)


@pytest.mark.parametrize("gate,l2", [("g", True), ("raw", False)])
def test_prior_buffer_contents_do_not_matter(gate, l2):
    # 0xFF bytes are NaN in bf16 and fp32: any read of an unwritten element shows.
    w = I.custom([130, 64, 1, 77], 3, gate=gate, l2norm=l2, seed=21, name="poison")
    print(f"[case] poisoned buffers {w.key} docs={w.doc_lens}", flush=True)
    dev = to_device(I.make_inputs(w))
    a = _poison_run(w, dev, 0x00)
    b = _poison_run(w, dev, 0xFF)
    for k in a:
        assert torch.isfinite(b[k].float()).all(), f"{k}: non-finite output after poisoning"
        assert _same_bits(a[k], b[k]), f"{k}: depends on prior buffer contents"


def test_document_isolation():
    w = I.custom([300, 700, 129], 2, gate="g", seed=22, name="iso")
    print(f"[case] isolation docs={w.doc_lens}", flush=True)
    inp = I.make_inputs(w)
    dev = to_device(inp)
    o1, g1, _ = run_gpu(w, dev)
    ref = {k: v.clone() for k, v in _outputs(o1, g1).items()}
    # perturb every input of the middle document
    lo, hi = 300, 1000
    dev2 = {k: v.clone() for k, v in dev.items()}
    for key in ("q", "k", "v", "dO"):
        dev2[key][lo:hi] = torch.flip(dev2[key][lo:hi], dims=[-1])
    dev2["beta"][lo:hi] = 0.25
    dev2["gate"][lo:hi] = dev2["gate"][lo:hi] * 3.0
    o2, g2, _ = run_gpu(w, dev2)
    got = _outputs(o2, g2)
    for k, v in got.items():
        for a, b in ((0, lo), (hi, w.T)):
            assert _same_bits(ref[k][a:b], v[a:b]), f"{k}: tokens {a}:{b} changed"
        assert not _same_bits(ref[k][lo:hi], v[lo:hi]), f"{k}: perturbation had no effect"


RAGGED = [
    ("g", False, [1, 63, 64, 65, 0, 127, 128, 129, 2]),
    ("raw", True, [65, 0, 0, 191, 1, 64]),
    ("g", True, [4096]),
]


@pytest.mark.parametrize("gate,l2,docs", RAGGED)
def test_ragged_and_empty_documents(gate, l2, docs):
    w = I.custom(docs, 2, gate=gate, l2norm=l2, seed=23, name="ragged")
    print(f"[case] ragged {w.key} docs={w.doc_lens}", flush=True)
    inp = I.make_inputs(w)
    dev = to_device(inp)
    o, g, _ = run_gpu(w, dev)
    oref, gref = run_oracle(w, inp)
    errs = {"o": rel_l2(f64(o), oref)}
    gg = gpu_grads_f64(w, g)
    errs.update({k: rel_l2(gg[k], v) for k, v in gref.items()})
    print("[parity] ragged " + ", ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL[k]}
    assert not bad, bad


def test_many_short_documents():
    # > 256 documents exercises the chunk map's multi-pass prefix sum
    rng = np.random.default_rng(5)
    docs = [int(x) for x in rng.integers(0, 90, size=700)]
    w = I.custom(docs, 1, gate="raw", seed=24, name="many")
    print(f"[case] many documents N={len(docs)} T={w.T}", flush=True)
    inp = I.make_inputs(w)
    dev = to_device(inp)
    o, g, _ = run_gpu(w, dev)
    oref, gref = run_oracle(w, inp)
    errs = {"o": rel_l2(f64(o), oref)}
    gg = gpu_grads_f64(w, g)
    errs.update({k: rel_l2(gg[k], v) for k, v in gref.items()})
    print("[parity] many " + ", ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL[k]}
    assert not bad, bad


def test_inner_product_identities_full_size():
    # o is linear in v and (L2 off) in q, so sum<v,dv> = sum<q,dq> = sum<o,dO>.
    # With dO = o the right side is |o|^2, so rounding noise in the bf16
    # gradients averages out and a systematic error would show.
    w = I.BY_NAME["4doc"]
    print(f"[case] identities {w.key} with dO = o", flush=True)
    dev = to_device(I.make_inputs(w))
    kda = KDA(w.T, w.H, len(w.doc_lens), gate=w.gate, l2norm=w.l2norm)
    args = (dev["q"], dev["k"], dev["v"], dev["beta"], dev["gate"], dev["cu_seqlens"])
    o = kda.forward(*args, dev["A_log"], dev["dt_bias"])
    g = kda.backward(*args, o, dev["A_log"], dev["dt_bias"])
    torch.cuda.synchronize()
    od = float((o.double() ** 2).sum())
    vd = float((dev["v"].double() * g["dv"].double()).sum())
    qd = float((dev["q"].double() * g["dq"].double()).sum())
    print(f"[parity] identities |o|^2={od:.8e} <v,dv>={vd:.8e} <q,dq>={qd:.8e}", flush=True)
    assert abs(vd - od) <= 1e-3 * od
    assert abs(qd - od) <= 1e-3 * od
