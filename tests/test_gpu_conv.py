"""GPU parity of the width-4 causal conv1d + SiLU op (flashinfer PR #7176,
description: the conv halo + conv step of the KDA module forward) against its
FP64 oracle on the same seeded bits, plus bitwise determinism and the
fragment identity (a document split in two, the second fragment given the
first one's last 3 tokens as its halo, gives the unsplit output).

Bounds (relative L2, float64): 2e-3 on the bf16 outputs y, dx and dhalo
(rounding to bf16 alone costs ~1.66e-3); 1e-4 on the fp32 sums dw and db
(each a fixed-order fp32 sum over the tokens of fp32 products).
"""

import numpy as np
import pytest
import torch

from gpu_common import bf16_tensor, f64, rel_l2
from kda_chunked_amd import inputs as I
from kda_chunked_amd.binding import ConvSiLU
from oracle import conv_oracle as co

pytestmark = pytest.mark.gpu

TOL = {"y": 2e-3, "dx": 2e-3, "dhalo": 2e-3, "dw": 1e-4, "db": 1e-4}


def _dev(inp):
    out = {k: bf16_tensor(inp[k]) for k in ("x", "dy", "halo") if k in inp}
    out["w"] = torch.from_numpy(inp["w"]).cuda()
    if "b" in inp:
        out["b"] = torch.from_numpy(inp["b"]).cuda()
    out["cu"] = torch.from_numpy(inp["cu_seqlens"].astype(np.int32)).cuda()
    return out


def _run(w, dev):
    op = ConvSiLU(w.T, w.D, len(w.doc_lens), bias=w.bias, halo=w.halo)
    y = op.forward(dev["x"], dev["w"], dev["cu"], dev.get("b"), dev.get("halo"))
    g = op.backward(dev["x"], dev["w"], dev["cu"], dev["dy"], dev.get("b"), dev.get("halo"))
    torch.cuda.synchronize()
    return y, g


def _oracle(inp, cols=None):
    f = lambda a: I.bf16_to_f32(a).astype(np.float64)
    sel = (lambda a: np.ascontiguousarray(a[:, cols])) if cols is not None else (lambda a: a)
    x, dy = f(sel(inp["x"])), f(sel(inp["dy"]))
    w = inp["w"].astype(np.float64)[cols] if cols is not None else inp["w"].astype(np.float64)
    b = inp.get("b")
    b = None if b is None else (b.astype(np.float64)[cols] if cols is not None else b.astype(np.float64))
    halo = inp.get("halo")
    halo = None if halo is None else f(sel(halo))
    cu = inp["cu_seqlens"].astype(np.int64)
    y, _ = co.conv_silu_fwd(cu, x, w, b, halo)
    g = co.conv_silu_bwd(cu, x, w, dy, b, halo)
    return y, g


def _compare(tag, y, g, yref, gref, cols=None):
    sel = (lambda a: a[:, cols]) if cols is not None else (lambda a: a)
    errs = {"y": rel_l2(sel(f64(y)), yref), "dx": rel_l2(sel(f64(g["dx"])), gref["dx"]),
            "dw": rel_l2(f64(g["dw"])[cols] if cols is not None else f64(g["dw"]), gref["dw"])}
    if "db" in gref and "db" in g:
        errs["db"] = rel_l2(f64(g["db"])[cols] if cols is not None else f64(g["db"]), gref["db"])
    if "dhalo" in gref:
        errs["dhalo"] = rel_l2(sel(f64(g["dhalo"])), gref["dhalo"])
    print(f"[parity] {tag}: " + ", ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL[k]}
    assert not bad, f"{tag}: over tolerance {bad}"


@pytest.mark.parametrize("name", ["conv_tiny", "conv_ragged", "conv_narrow"])
def test_conv_parity_full(name):
    w = I.CONV_BY_NAME[name]
    print(f"[case] {name} T={w.T} D={w.D} docs={w.doc_lens}", flush=True)
    inp = I.make_conv_inputs(w)
    y, g = _run(w, _dev(inp))
    yref, gref = _oracle(inp)
    _compare(name, y, g, yref, gref)


def test_conv_parity_full_size_sampled_channels():
    """The 16384-token, 24576-channel workload the bench times; channels are
    independent, so the oracle recomputes every 48th channel."""
    w = I.CONV_BY_NAME["conv_4doc"]
    print(f"[case] conv_4doc T={w.T} D={w.D}", flush=True)
    inp = I.make_conv_inputs(w)
    y, g = _run(w, _dev(inp))
    cols = np.arange(0, w.D, 48)
    yref, gref = _oracle(inp, cols)
    _compare("conv_4doc (every 48th channel)", y, g, yref, gref, cols)


def test_conv_bitwise_deterministic():
    w = I.CONV_BY_NAME["conv_4doc"]
    dev = _dev(I.make_conv_inputs(w))
    y1, g1 = _run(w, dev)
    first = [y1.clone()] + [g1[k].clone() for k in sorted(g1)]
    y2, g2 = _run(w, dev)
    second = [y2] + [g2[k] for k in sorted(g2)]
    for a, b in zip(first, second):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.uint8) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.parametrize("m", [2, 101])
def test_conv_fragments_with_halo_equal_the_whole(m):
    """A 300-token document split after m tokens: the second fragment's halo
    is the 3 tokens before it (zero-padded); y matches the unsplit run bit for
    bit, and dw adds up."""
    D, n = 256, 300
    full = I.ConvWorkload("frag", (n,), D, True, False, seed=21)
    inp = I.make_conv_inputs(full)
    dev = _dev(inp)
    y, g = _run(full, dev)
    lead = torch.zeros(3, D, dtype=torch.bfloat16, device="cuda")
    k = min(m, 3)
    lead[3 - k:] = dev["x"][m - k:m]
    A = I.ConvWorkload("A", (m,), D, True, False)
    B = I.ConvWorkload("B", (n - m,), D, True, True)
    cuA = torch.tensor([0, m], dtype=torch.int32, device="cuda")
    cuB = torch.tensor([0, n - m], dtype=torch.int32, device="cuda")
    yA, gA = _run(A, dict(dev, x=dev["x"][:m].contiguous(), dy=dev["dy"][:m].contiguous(), cu=cuA))
    yB, gB = _run(B, dict(dev, x=dev["x"][m:].contiguous(), dy=dev["dy"][m:].contiguous(), cu=cuB,
                          halo=lead))
    assert torch.equal(torch.cat([yA, yB]).view(torch.uint8), y.view(torch.uint8))
    assert rel_l2(f64(gA["dw"]) + f64(gB["dw"]), f64(g["dw"])) < 1e-5
