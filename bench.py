"""Benchmark of the KDA training hot path on one MI355X.

One step = kda_fwd (writing the saved forward set) + kda_bwd (from it) over
the 1doc workload: one packed document of 16384 tokens, 64 heads, head dim
128, gate form g, Q/K L2 norm fused in the kernels, bf16 q/k/v/beta/dO and an
fp32 gate (the deterministic KDA package's timing row 1doc:g:fused:saved on
flashinfer PR #8909, timing tables). Inputs are seeded synthetic data that is
resident in HBM before the timed region starts.

Prints one JSON line: throughput in tokens/s (packed tokens x all heads per
step), the roofline of the dominant kernel (timed live with HIP events on
the stream the library launches on, through the library's launch hook), and
the FP64 oracle timed on the host on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload 1doc]
                       [--no-cpu] [--extra]
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0

# Algorithmic multiply-adds per full 64-token chunk and head, per kernel: the
# products the method defines (triangular products counted on their nonzero
# half), not the executed split terms.
_TRI = 64 * 65 // 2 * 128          # lower triangle incl. diagonal, K = 128
_TRI_S = 64 * 63 // 2 * 128        # strictly lower
_SQ = 64 * 128 * 128               # 64 x 128 x 128
MAC_PER_CHUNK_HEAD = {
    "fwd_prep": _TRI_S + _TRI + 64 ** 3 // 6,
    "fwd_scan": 3 * _SQ + 2 * _TRI,
    "bwd_scan": 3 * _SQ + 2 * _TRI,
    "bwd_intra": 3 * _SQ + 6 * _TRI + 2 * _TRI_S + 64 ** 3 // 2,
}


class HipEvents:
    """Per-kernel HIP event pairs recorded from the library's launch hook."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.records = []      # (kernel, start_event, end_event)
        self.open = {}

    def _event(self):
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def hook(self, name, end, stream):
        ev = self._event()
        if self.hip.hipEventRecord(ev, ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")
        if not end:
            self.open[name] = ev
        else:
            self.records.append((name, self.open.pop(name), ev))

    def durations_ms(self):
        out = {}
        for name, a, b in self.records:
            self.hip.hipEventSynchronize(b)
            ms = ctypes.c_float()
            self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
            out.setdefault(name, []).append(ms.value)
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)
        self.records = []
        return out


def make_device_inputs(w, torch):
    import numpy as np
    from kda_chunked_amd import inputs as I
    inp = I.make_inputs(w)
    dev = {}
    for key in ("q", "k", "v", "beta", "dO"):
        dev[key] = torch.from_numpy(inp[key].view(np.int16)).view(torch.bfloat16).cuda()
    g = inp["gate"]
    dev["gate"] = (torch.from_numpy(g.view(np.int16)).view(torch.bfloat16)
                   if g.dtype == np.uint16 else torch.from_numpy(g)).cuda()
    for key in ("A_log", "dt_bias"):
        if key in inp:
            dev[key] = torch.from_numpy(inp[key]).cuda()
    dev["cu"] = torch.from_numpy(inp["cu_seqlens"]).cuda()
    return inp, dev


def cpu_baseline(w, inp, threads):
    """The FP64 oracle (as it stands) on a bounded sample of the workload:
    2 heads per host thread of the same document(s), fwd + bwd."""
    import numpy as np
    from kda_chunked_amd import inputs as I
    from oracle import kda_oracle as ko
    nh = min(w.H, 2 * threads)
    hs = list(range(nh))
    f = I.as_f64({k: (v[:, hs] if k in ("q", "k", "v", "beta", "dO", "gate") else v)
                  for k, v in inp.items()})
    extra = {}
    if w.gate == "raw":
        extra = dict(A_log=f["A_log"][hs], dt_bias=f["dt_bias"][hs])
    t = time.perf_counter()
    ko.fwd(f["cu_seqlens"], f["q"], f["k"], f["v"], f["beta"], f["gate"], gate_form=w.gate,
           l2norm=w.l2norm, threads=threads, **extra)
    ko.bwd(f["cu_seqlens"], f["q"], f["k"], f["v"], f["beta"], f["gate"], f["dO"],
           gate_form=w.gate, l2norm=w.l2norm, threads=threads, **extra)
    sec = time.perf_counter() - t
    tokens = w.T * nh / w.H          # whole-token equivalents (all heads)
    return {"value": tokens / sec, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{w.name}: {w.T} tokens x {nh} of {w.H} heads, fwd+bwd, "
                      f"{sec:.1f} s on {threads} threads; value scaled to all heads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="1doc")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--extra", action="store_true", help="also time fwd and bwd alone")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this build runs on one GPU "
              "(heads or sequence shards would split across GPUs; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from kda_chunked_amd import inputs as I
    from kda_chunked_amd.binding import KDA, lib, set_launch_hook

    lib()
    w = I.BY_NAME[args.workload]
    inp, dev = make_device_inputs(w, torch)
    kda = KDA(w.T, w.H, len(w.doc_lens), gate=w.gate, l2norm=w.l2norm)
    A_log, dt_bias = dev.get("A_log"), dev.get("dt_bias")
    grads = dict(dq=torch.empty_like(dev["q"]), dk=torch.empty_like(dev["k"]),
                 dv=torch.empty_like(dev["v"]), dbeta=torch.empty_like(dev["beta"]),
                 dgate=torch.empty_like(dev["gate"]))
    if w.gate == "raw":
        grads.update(dA_log=torch.empty_like(A_log), ddt_bias=torch.empty_like(dt_bias))
    o = torch.empty_like(dev["v"])

    def fwd():
        kda.forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["gate"], dev["cu"], A_log,
                    dt_bias, save=True, o=o)

    def bwd():
        kda.backward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["gate"], dev["cu"],
                     dev["dO"], A_log, dt_bias, out=grads)

    def step():
        fwd()
        bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, per-kernel HIP events from the hook
    ev = HipEvents()
    set_launch_hook(ev.hook)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    set_launch_hook(None)
    ms_step = start.elapsed_time(stop) / args.steps
    kern = ev.durations_ms()
    kern_avg = {k: statistics.fmean(v) for k, v in kern.items()}

    extra = {}
    if args.extra:
        for name, fn in (("fwd", fwd), ("bwd", bwd)):
            samples = []
            for _ in range(5):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(5):
                    fn()
                b.record()
                torch.cuda.synchronize()
                samples.append(a.elapsed_time(b) / 5)
            extra[f"{name}_ms"] = round(statistics.median(samples), 4)

    units = w.T * w.H / 64.0    # chunk-head equivalents per launch
    dom = max((k for k in kern_avg if k in MAC_PER_CHUNK_HEAD), key=lambda k: kern_avg[k])
    flop = 2.0 * MAC_PER_CHUNK_HEAD[dom] * units
    achieved = flop / (kern_avg[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "algorithmic_flop_per_launch": flop, "avg_launch_ms": round(kern_avg[dom], 4)}

    total_flop = 2.0 * sum(MAC_PER_CHUNK_HEAD.values()) * units
    line = {
        "metric": "KDA fwd+bwd tokens/s (16384 tok x 64 heads, d=128)",
        "value": round(w.T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.key + ":saved", "tokens": w.T, "heads": w.H, "head_dim": 128,
                   "docs": list(w.doc_lens), "chunk": 64},
        "roofline": roofline,
        "kernels_ms": {k: round(v, 4) for k, v in sorted(kern_avg.items())},
        "algorithmic_tflops": round(total_flop / (ms_step * 1e-3) / 1e12, 2),
        "wall_s_timed": round(wall, 3),
    }
    line.update(extra)
    if not args.no_cpu:
        from oracle import kda_oracle as ko
        line["cpu_baseline"] = cpu_baseline(w, inp, ko.default_threads())
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
