"""kda_fwd_noalloc against kda_fwd on the GPU: the forward without a workspace
argument (the library's fixed per-GPU scratch serves instead) must give the
same o and the same saved set as the forward with a caller workspace, so the
backward from either saved set is bitwise the same. Two calls in a row, the
second on a smaller problem, and a non-saving call whose per-chunk set fits
the scratch. Bitwise equality is stronger than the oracle tolerance: both
calls run the same kernels on the same inputs (flashinfer PR #8909, opening
section: bitwise reproducible forward and backward)."""

import pytest
import torch

from gpu_common import to_device
from kda_chunked_amd import binding as B
from kda_chunked_amd import inputs as I

pytestmark = pytest.mark.gpu


def _same_bits(a, b):
    return a.shape == b.shape and torch.equal(a.contiguous().view(torch.uint8),
                                              b.contiguous().view(torch.uint8))


def _grads(kda, dev, saved):
    out = dict(dq=torch.empty_like(dev["q"]), dk=torch.empty_like(dev["k"]),
               dv=torch.empty_like(dev["v"]), dbeta=torch.empty_like(dev["beta"]),
               dgate=torch.empty_like(dev["gate"]))
    if kda.gate == "raw":
        out.update(dA_log=torch.empty_like(dev["A_log"]), ddt_bias=torch.empty_like(dev["dt_bias"]))
    B.kda_bwd(kda.p, dev["q"], dev["k"], dev["v"], dev["beta"], dev["gate"], dev.get("A_log"),
              dev.get("dt_bias"), dev["cu_seqlens"], dev["dO"], saved, out["dq"], out["dk"],
              out["dv"], out["dbeta"], out["dgate"], out.get("dA_log"), out.get("ddt_bias"),
              kda.workspace)
    return out


@pytest.mark.parametrize("names", [("R2", "tiny")])
def test_noalloc_forward_matches_kda_fwd(names):
    for name in names:                      # two calls in a row, the second smaller
        w = I.BY_NAME[name]
        print(f"[case] no-alloc forward {w.key} T={w.T} H={w.H}", flush=True)
        dev = to_device(I.make_inputs(w))
        kda = B.KDA(w.T, w.H, len(w.doc_lens), gate=w.gate, l2norm=w.l2norm)
        args = (dev["q"], dev["k"], dev["v"], dev["beta"], dev["gate"], dev.get("A_log"),
                dev.get("dt_bias"), dev["cu_seqlens"])
        o_ref = torch.empty_like(dev["v"])
        B.kda_fwd(kda.p, *args, o_ref, kda.saved, kda.workspace)
        g_ref = _grads(kda, dev, kda.saved)
        o_na = torch.full_like(dev["v"], float("nan"))
        saved_na = torch.empty_like(kda.saved)
        B.kda_fwd_noalloc(kda.p, *args, o_na, saved_na)
        g_na = _grads(kda, dev, saved_na)
        torch.cuda.synchronize()
        assert _same_bits(o_na, o_ref), f"{name}: o differs"
        for k, v in g_ref.items():
            assert _same_bits(g_na[k], v), f"{name}: {k} from the no-alloc saved set differs"
        if B.workspace_bytes(kda.p, False, True) <= B.NOALLOC_SCRATCH_BYTES:
            # no saved set: the per-chunk set lives in the scratch
            o_ns = torch.full_like(dev["v"], float("nan"))
            B.kda_fwd_noalloc(kda.p, *args, o_ns, None)
            torch.cuda.synchronize()
            assert _same_bits(o_ns, o_ref), f"{name}: non-saving o differs"
        else:
            with pytest.raises(B.KdaError) as e:
                B.kda_fwd_noalloc(kda.p, *args, torch.empty_like(dev["v"]), None)
            assert e.value.status == 3
