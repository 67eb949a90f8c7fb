"""Stream behaviour of the C ABI on the GPU: calls are only enqueued (the host
never waits for the device), they run on the caller's stream, a kernel resident
on another stream does not change their results, and a zero-token raw backward
writes its zero parameter gradients.

These are the boundary conventions the library borrows from the packed-varlen
GQA training op (flashinfer PR #7774, description and commit notes: no device
synchronisation, a resident side-stream kernel, launch on the operand device's
current stream); results must be bitwise those of a run on the default stream
(flashinfer PR #8909, opening section: bitwise reproducible).
"""

import pytest
import torch

from gpu_common import run_gpu, to_device
from kda_chunked_amd import inputs as I
from kda_chunked_amd.binding import KDA

pytestmark = pytest.mark.gpu

W = I.BY_NAME["m2"]


def _same_bits(a, b):
    return a.shape == b.shape and torch.equal(a.contiguous().view(torch.uint8),
                                              b.contiguous().view(torch.uint8))


def _busy(x, n):
    """Enqueue n in-place passes over x (a long but finite stream of work)."""
    for _ in range(n):
        x.mul_(1.0000001)


def _reference(dev):
    o, g, _ = run_gpu(W, dev)
    return o.clone(), {k: v.clone() for k, v in g.items() if v is not None}


def test_calls_do_not_synchronise_and_use_the_callers_stream():
    dev = to_device(I.make_inputs(W))
    o_ref, g_ref = _reference(dev)
    kda = KDA(W.T, W.H, len(W.doc_lens), gate=W.gate, l2norm=W.l2norm)
    side = torch.cuda.Stream()
    filler = torch.ones(1 << 26, device="cuda")     # 256 MiB
    torch.cuda.synchronize()
    print("[case] no host synchronisation, non-default stream", flush=True)
    with torch.cuda.stream(side):
        _busy(filler, 400)                          # queued ahead of the KDA calls
        o = kda.forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["gate"],
                        dev["cu_seqlens"])
        g = kda.backward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["gate"],
                         dev["cu_seqlens"], dev["dO"])
        still_busy = not side.query()
    side.synchronize()
    assert still_busy, "the calls returned after the stream had drained: the host waited"
    assert _same_bits(o, o_ref)
    for k, v in g_ref.items():
        assert _same_bits(g[k], v), k


def test_resident_side_stream_kernel_does_not_change_results():
    dev = to_device(I.make_inputs(W))
    o_ref, g_ref = _reference(dev)
    side = torch.cuda.Stream()
    filler = torch.ones(1 << 26, device="cuda")
    torch.cuda.synchronize()
    print("[case] resident side-stream kernel", flush=True)
    with torch.cuda.stream(side):
        _busy(filler, 400)
    o, g, _ = run_gpu(W, dev)                       # default stream, concurrently
    side.synchronize()
    assert _same_bits(o, o_ref)
    for k, v in g_ref.items():
        assert _same_bits(g[k], v), k


def test_zero_tokens_raw_backward_zeroes_parameter_gradients():
    from kda_chunked_amd import binding as B
    p = B.problem(0, 3, 1, gate="raw")
    dA_log = torch.full((3,), float("nan"), device="cuda")
    ddt_bias = torch.full((3, 128), float("nan"), device="cuda")
    t = torch.zeros(16, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(max(B.workspace_bytes(p, True, True), 16), dtype=torch.uint8, device="cuda")
    print("[case] T = 0 raw backward", flush=True)
    B.kda_bwd(p, t, t, t, t, t, t, t, t, t, None, t, t, t, t, t, dA_log, ddt_bias, ws)
    torch.cuda.synchronize()
    assert torch.all(dA_log == 0) and torch.all(ddt_bias == 0)
