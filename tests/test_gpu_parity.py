"""GPU parity: the HIP path against the FP64 oracle on the same seeded bits.

Every workload is compared on every element: tiny, m2 and R2, and the two
16384-token, 64-head workloads at full size in the configuration the bench
times (1doc saved; 4doc saved and replay), where the worst (document, head)
slice is bounded as well as the whole tensor.

Bounds (relative L2 over the tensor, float64): 2e-3 for o, dq, dk, dv, dbeta
(bf16 outputs; rounding alone costs ~1.66e-3), 1e-2 for the gate gradients.
"""

import numpy as np
import pytest
import torch

from gpu_common import (TOL, bf16_floor, gpu_grads_f64, rel_l2, run_gpu, run_oracle,
                        to_device, f64)
from kda_chunked_amd import inputs as I

pytestmark = pytest.mark.gpu


def _report(tag, errs):
    print(f"[parity] {tag}: " + ", ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)


def _compare(w, tag, o, g, oref, gref, heads=None):
    hs = slice(None) if heads is None else list(heads)
    errs = {"o": rel_l2(f64(o)[:, hs], oref)}
    gg = gpu_grads_f64(w, g)
    for name, ref in gref.items():
        x = gg[name]
        if name in ("dA_log", "ddt_bias"):
            x = x[hs]
        else:
            x = x[:, hs]
        errs[name] = rel_l2(x, ref)
    _report(tag, errs)
    print(f"[parity] {tag}: bf16 floor of o = {bf16_floor(oref):.3e}", flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL[k]}
    assert not bad, f"{tag}: over tolerance {bad}"


@pytest.mark.parametrize("name", ["tiny", "m2", "R2"])
def test_parity_full(name):
    w = I.BY_NAME[name]
    inp = I.make_inputs(w)
    print(f"[case] {w.key} T={w.T} H={w.H} docs={w.doc_lens}", flush=True)
    dev = to_device(inp)
    o, g, _ = run_gpu(w, dev)
    oref, gref = run_oracle(w, inp)
    _compare(w, w.key, o, g, oref, gref)


_ORACLE = {}


def _oracle_all_heads(w, inp):
    """Oracle results of a workload on every head (cached: the saved and the
    replay backward compute the same function)."""
    if w.name not in _ORACLE:
        _ORACLE.clear()
        _ORACLE[w.name] = run_oracle(w, inp)
    return _ORACLE[w.name]


def _slice_errors(w, o, gg, oref, gref):
    """Largest relative L2 error over every (document, head) slice, per tensor."""
    cu = w.cu_seqlens
    worst = {}
    tensors = {"o": (o, oref)}
    tensors.update({k: (gg[k], v) for k, v in gref.items() if k not in ("dA_log", "ddt_bias")})
    for name, (x, ref) in tensors.items():
        m = 0.0
        for d in range(len(w.doc_lens)):
            a, b = int(cu[d]), int(cu[d + 1])
            for h in range(w.H):
                m = max(m, rel_l2(x[a:b, h], ref[a:b, h]))
        worst[name] = m
    return worst


@pytest.mark.parametrize("name,replay", [("1doc", False), ("4doc", False), ("4doc", True)])
def test_parity_full_size_all_heads(name, replay):
    """Every head of the 16384-token, 64-head workloads, run in the bench's
    launch configuration: whole-tensor relative L2 and the worst (document,
    head) slice, both under the same bounds."""
    w = I.BY_NAME[name]
    inp = I.make_inputs(w)
    tag = f"{w.key}:{'replay' if replay else 'saved'}"
    print(f"[case] {tag} T={w.T} H={w.H} all heads", flush=True)
    dev = to_device(inp)
    o, g, _ = run_gpu(w, dev, replay=replay)
    oref, gref = _oracle_all_heads(w, inp)
    o64, gg = f64(o), gpu_grads_f64(w, g)
    errs = {"o": rel_l2(o64, oref)}
    errs.update({k: rel_l2(gg[k], v) for k, v in gref.items()})
    _report(tag, errs)
    worst = _slice_errors(w, o64, gg, oref, gref)
    _report(tag + " worst (document, head) slice", worst)
    bad = {k: v for k, v in errs.items() if not v <= TOL[k]}
    bad.update({k + "[slice]": v for k, v in worst.items() if not v <= TOL[k]})
    assert not bad, f"{tag}: over tolerance {bad}"


def _saved_states(kda, w):
    """The S_in block of the saved set (layout: Tm, Akk, rq, rk, S_in, ...,
    each 256-byte aligned). S_in is stored in MFMA tile order: tile (rb, cb) of
    16 x 16 at (8 rb + cb) * 256 floats, element (4 g + i, c) of the tile at
    4 (16 g + c) + i."""
    up = lambda x: (x + 255) // 256 * 256
    NC = w.T // 64 + len(w.doc_lens)
    H, T = w.H, w.T
    off = 2 * up(NC * H * 4096 * 4) + 2 * up(T * H * 4)
    n = NC * H * 128 * 128
    raw = kda.saved[off:off + 4 * n].view(torch.float32).view(NC, H, 8, 8, 4, 16, 4)
    return raw.permute(0, 1, 2, 4, 6, 3, 5).reshape(NC, H, 128, 128)


@pytest.mark.parametrize("name", ["tiny", "m2"])
def test_saved_states_match_oracle(name):
    from oracle import kda_oracle as ko
    w = I.BY_NAME[name]
    inp = I.make_inputs(w)
    dev = to_device(inp)
    _, _, kda = run_gpu(w, dev)
    f = I.as_f64(inp)
    _, S = ko.fwd(f["cu_seqlens"], f["q"], f["k"], f["v"], f["beta"], f["gate"], chunk=64,
                  gate_form=w.gate, l2norm=w.l2norm)
    got = f64(_saved_states(kda, w))[: S.shape[0]]
    err = rel_l2(got, S)
    print(f"[parity] {w.key}: saved S_in rel-L2 {err:.3e}", flush=True)
    assert err < 1e-3
