"""Helpers shared by the GPU tests: moving seeded inputs to the device,
running the library, running the oracle on the same bits, and tolerances."""

from __future__ import annotations

import numpy as np
import torch

from kda_chunked_amd import inputs as I

# relative L2 bounds (whole tensor, float64): bf16 outputs and the fp32 gate gradient
TOL = {"o": 2e-3, "dq": 2e-3, "dk": 2e-3, "dv": 2e-3, "dbeta": 2e-3,
       "dg": 1e-2, "da": 1e-2, "dA_log": 1e-2, "ddt_bias": 1e-2}


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_device(inp: dict, device="cuda") -> dict:
    out = {}
    for key in ("q", "k", "v", "beta", "dO"):
        out[key] = bf16_tensor(inp[key], device)
    g = inp["gate"]
    out["gate"] = bf16_tensor(g, device) if g.dtype == np.uint16 else torch.from_numpy(g).to(device)
    for key in ("A_log", "dt_bias"):
        if key in inp:
            out[key] = torch.from_numpy(inp[key]).to(device)
    out["cu_seqlens"] = torch.from_numpy(inp["cu_seqlens"].astype(np.int32)).to(device)
    return out


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_gpu(w: I.Workload, dev: dict, replay=False, kda=None):
    """Forward (saving unless replay) then backward. Returns (o, grads, kda)."""
    from kda_chunked_amd.binding import KDA
    if kda is None:
        kda = KDA(w.T, w.H, len(w.doc_lens), gate=w.gate, l2norm=w.l2norm)
    o = kda.forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["gate"], dev["cu_seqlens"],
                    dev.get("A_log"), dev.get("dt_bias"), save=not replay)
    g = kda.backward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["gate"], dev["cu_seqlens"],
                     dev["dO"], dev.get("A_log"), dev.get("dt_bias"), replay=replay)
    torch.cuda.synchronize()
    return o, g, kda


def gpu_grads_f64(w: I.Workload, g: dict) -> dict:
    out = {"dq": f64(g["dq"]), "dk": f64(g["dk"]), "dv": f64(g["dv"]), "dbeta": f64(g["dbeta"])}
    if w.gate == "raw":
        out.update(da=f64(g["dgate"]), dA_log=f64(g["dA_log"]), ddt_bias=f64(g["ddt_bias"]))
    else:
        out["dg"] = f64(g["dgate"])
    return out


def run_oracle(w: I.Workload, inp: dict, heads=None):
    """Oracle forward and backward on the same bits (optionally a subset of heads)."""
    from oracle import kda_oracle as ko
    f = I.as_f64(inp)
    hs = list(range(w.H)) if heads is None else list(heads)
    sel = lambda a: np.ascontiguousarray(a[:, hs])
    args = (f["cu_seqlens"], sel(f["q"]), sel(f["k"]), sel(f["v"]), sel(f["beta"]), sel(f["gate"]))
    extra = {}
    if w.gate == "raw":
        extra = dict(A_log=f["A_log"][hs], dt_bias=f["dt_bias"][hs])
    o = ko.fwd(*args, gate_form=w.gate, l2norm=w.l2norm, **extra)
    g = ko.bwd(*args, sel(f["dO"]), gate_form=w.gate, l2norm=w.l2norm, **extra)
    return o, g


def rel_l2(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))


def bf16_floor(ref):
    r32 = np.asarray(ref, np.float32)
    return rel_l2(I.bf16_to_f32(I.f32_to_bf16(r32)), ref)
