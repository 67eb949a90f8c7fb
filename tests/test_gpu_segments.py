"""Segment-parallel scans on the GPU: with few chains (documents x heads x 4
column tiles below 192) the library cuts each document into segments, runs the
state scans on all segments at once from their FP32 affine summaries
S_out = M S_in + B and the transfer walk between them (flashinfer PR #7176,
opening section), and the reverse scan likewise through dS_in = M^T dS_out + B'.
These cases put documents of 1 to 6 segments, and documents shorter than one
segment, beside each other, and compare every output with the FP64 oracle;
saved and replay backward must stay bitwise equal and reproducible."""

import pytest
import torch

from gpu_common import TOL, f64, gpu_grads_f64, rel_l2, run_gpu, run_oracle, to_device
from kda_chunked_amd import inputs as I

pytestmark = pytest.mark.gpu

CASES = [
    # (docs, H, gate, l2): segments of 16 chunks (documents average at least two)
    ((6000, 70, 1030), 1, "g", False),      # 6, 1 and 2 segments
    ((4000, 1300), 2, "raw", False),        # 4 and 2 segments
    ((5000,), 2, "g", True),                # 5 segments
]


@pytest.mark.parametrize("docs,H,gate,l2", CASES, ids=["g-3doc-H1", "raw-2doc-H2", "g-l2-1doc-H2"])
def test_segmented_scans_match_oracle(docs, H, gate, l2):
    w = I.custom(docs, H, gate=gate, l2norm=l2, seed=41, name="seg")
    print(f"[case] segments {w.key} docs={w.doc_lens} H={H}", flush=True)
    inp = I.make_inputs(w)
    dev = to_device(inp)
    o, g, kda = run_gpu(w, dev)
    oref, gref = run_oracle(w, inp)
    gg = gpu_grads_f64(w, g)
    errs = {"o": rel_l2(f64(o), oref)}
    errs.update({k: rel_l2(gg[k], v) for k, v in gref.items()})
    print("[parity] segments " + ", ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL[k]}
    assert not bad, bad
    # replay (forward recomputed, walks included) is bitwise the saved backward
    saved = {k: v.clone() for k, v in g.items() if v is not None}
    _, gr, _ = run_gpu(w, dev, replay=True, kda=kda)
    for k, v in saved.items():
        assert torch.equal(v.view(torch.uint8), gr[k].view(torch.uint8)), k
