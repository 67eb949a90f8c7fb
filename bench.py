"""Benchmark of the KDA training hot path on one MI355X.

One step = kda_fwd (writing the saved forward set) + kda_bwd (from it) over
the 1doc workload: one packed document of 16384 tokens, 64 heads, head dim
128, gate form g, Q/K L2 norm fused in the kernels, bf16 q/k/v/beta/dO and an
fp32 gate (the deterministic KDA package's timing row 1doc:g:fused:saved on
flashinfer PR #8909, timing tables). Inputs are seeded synthetic data that is
resident in HBM before the timed region starts.

Prints one JSON line: throughput in tokens/s (packed tokens x all heads per
step); the roofline of the dominant contraction kernel (the longest MFMA
kernel of the step, timed live with HIP events on the stream the library
launches on, through the library's launch hook) as its algorithmic FLOP rate
against the dense bf16 MFMA peak, with its compulsory HBM bytes and the
measured HBM traffic beside it; the whole step on the method's own work and
compulsory bytes; and the FP64 oracle timed on the host on a bounded sample of
the same workload.

Besides the timed steps it times, outside the timed region, the units of the
deterministic package's protocol: fwd alone, bwd alone and the replay pair
(forward without saving, backward recomputing the forward), each the median
of 15 samples of 20 back-to-back calls; the same units for the package's
other timing rows that this repository reproduces (4doc saved and replay, R2,
m2); the conv1d + SiLU op that precedes the state passing; and the packed-varlen
causal GQA attention of the same family (2 x forward + backward), as extra keys.

HBM traffic and MFMA utilisation come from rocprofv3 counter runs whose
summaries sit in profiles/; they are reported only while the kernel sources
still hash to the fingerprint recorded with them (else null).

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload 1doc]
                       [--no-cpu] [--no-units] [--no-rows] [--calibrate-copy MIB]
       python bench.py --pmc-summary DIR     (tabulate a rocprofv3 --pmc run)
       python bench.py --trace-summary DIR   (tabulate a rocprofv3 --kernel-trace run)
       python bench.py --fingerprint         (hash of the kernel sources)
"""

from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "KDA fwd+bwd ms & tokens/s, 16384 tok x 64 heads, d=128; MFMA util %"
CSRC = os.path.join(ROOT, "kda_chunked_amd", "csrc")
# fwd+bwd ms per row on NVIDIA GB300 ("after head" column of the GB300 timing
# table on flashinfer PR #8909): another machine's numbers, context only.
PAGE_FWD_BWD_MS = {"1doc:g:fused": 4.4696, "4doc:raw:off": 4.2789,
                   "4doc:raw:off:replay": 5.0539, "R2:raw:off": 0.6658, "m2:g:off": 0.5285}
PROFILES = os.path.join(ROOT, "profiles")

# Algorithmic multiply-adds per full 64-token chunk and head, per kernel: the
# products the method defines (triangular products counted on their nonzero
# half), not the executed split terms.
_TRI = 64 * 65 // 2 * 128          # lower triangle incl. diagonal, K = 128
_TRI_S = 64 * 63 // 2 * 128        # strictly lower
_SQ = 64 * 128 * 128               # 64 x 128 x 128
MAC_PER_CHUNK_HEAD = {
    "fwd_prep": _TRI_S + _TRI + 64 ** 3 // 6,
    "fwd_scan": 2 * _SQ + _TRI,        # R = V - Kd S_in, U~ = Tb R, Ke^T U~
    "fwd_out": _SQ + _TRI,             # Qd S_in, A_qk U~
    "bwd_scan": 3 * _SQ + 2 * _TRI,
    "bwd_intra": 3 * _SQ + 6 * _TRI + 2 * _TRI_S + 64 ** 3 // 2,
}

# Algorithmic bytes per full chunk and head, per kernel: every tensor the
# kernel reads or writes in this design's data flow, counted once at its
# stored precision (a panel read by several workgroups counts once). Gate
# form g stores an fp32 g / dg; the raw form a bf16 a / da plus fp32 partials.
_X = 64 * 128                      # elements of a 64 x 128 per-chunk tensor
_PANEL_B = 131584                  # operand panels (bf16 hi/lo planes), read by all three scans
_FWD_CHAIN_B = 57856               # their chain part: -Kd, Tb, Ke^T hi/lo, e^(G_last)


def algo_bytes_per_chunk_head(kernel: str, raw: bool) -> int:
    gate_in = 2 * _X if raw else 4 * _X            # a (bf16) or g (fp32)
    gate_out = 2 * _X + 512 + 4 if raw else 4 * _X  # da + part_dt + part_A, or dg
    return {
        # q, k, gate, beta -> rq, rk, T, A_kk, operand panels
        "fwd_prep": 2 * 2 * _X + gate_in + 128 + 512 + 2 * 4 * 64 * 64 + _PANEL_B,
        # chain panels, v -> S_in, R, U~ (fp32)
        "fwd_scan": _FWD_CHAIN_B + 2 * _X + 4 * 128 * 128 + 2 * 4 * _X,
        # S_in, U~, scale Qd, scale A_qk -> o
        "fwd_out": 4 * 128 * 128 + 4 * _X + 2 * 2 * _X + 2 * 2 * 64 * 64 + 2 * _X,
        # panels, dO -> dv, dU~ (fp32), dS (fp32)
        "bwd_scan": _PANEL_B + 2 * _X + 2 * _X + 4 * _X + 4 * 128 * 128,
        # q, k, gate, dO, dv, beta, rq, rk, S_in, dS, U~, R, dU~, T, A_kk
        # -> dq, dk, dbeta, dgate
        "bwd_intra": 2 * 2 * _X + gate_in + 2 * _X + 2 * _X + 128 + 512 + 2 * 4 * 128 * 128
                     + 3 * 4 * _X + 2 * 4 * 64 * 64 + 2 * 2 * _X + 128 + gate_out,
    }[kernel]


# The method's own work and compulsory HBM traffic per token-head (one token
# of one head), independent of this design's intermediates:
# * FLOP: a full 64-token chunk-head takes 4.51 M multiply-adds forward
#   (A_kk 0.26 M, A_qk 0.27 M, UT solve 0.04 M, W 0.27 M, U 0.27 M, W S 1.05 M,
#   K_dec^T U~ 1.05 M, O 1.31 M) and 11.17 M backward (reverse state scan
#   3.41 M, intra-chunk gradients 5.6 M, recomputing A_kk, A_qk, T and U~
#   2.15 M): 141 k + 349 k FLOP per token-head.
# * Bytes: every input read once and every output written once at its storage
#   precision. Gate form g: forward reads q, k, v (bf16), beta (bf16), g (fp32)
#   and writes o; backward reads those and dO and writes dq, dk, dv, dbeta, dg.
#   The raw form replaces the fp32 g / dg with a bf16 a / da (A_log, dt_bias
#   and their gradients are per head, negligible).
FLOP_PER_TOKEN_HEAD = {"fwd": 2 * 4.51e6 / 64, "bwd": 2 * 11.17e6 / 64}
COMPULSORY_BYTES_PER_TOKEN_HEAD = {
    False: {"fwd": 3 * 256 + 2 + 512 + 256, "bwd": 3 * 256 + 2 + 512 + 256 + 3 * 256 + 2 + 512},
    True: {"fwd": 3 * 256 + 2 + 256 + 256, "bwd": 3 * 256 + 2 + 256 + 256 + 3 * 256 + 2 + 256},
}
# The per-chunk backward's own compulsory I/O: q, k, gate, beta, dO in;
# dq, dk, dbeta, dgate out (dv leaves the reverse scan).
BWD_INTRA_COMPULSORY_BYTES_PER_TOKEN_HEAD = {
    False: 256 + 256 + 512 + 2 + 256 + 256 + 256 + 2 + 512,
    True: 256 + 256 + 256 + 2 + 256 + 256 + 256 + 2 + 256,
}
MFMA_KERNELS = ("fwd_prep", "fwd_scan", "fwd_out", "bwd_scan", "bwd_intra")


def kernel_roofline(kernel: str, ms: float, chunk_heads: float, raw: bool) -> dict:
    """A contraction kernel against the dense bf16 MFMA peak: its algorithmic
    FLOP per launch (the method's products, triangles on their nonzero half,
    split terms not counted) over its average launch time. The HBM view of the
    same launch (this design's stored bytes at 8 TB/s) is secondary."""
    flop = 2.0 * MAC_PER_CHUNK_HEAD[kernel] * chunk_heads
    nbytes = float(algo_bytes_per_chunk_head(kernel, raw)) * chunk_heads
    ach = flop / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
            "algorithmic_flop_per_launch": flop, "design_bytes_per_launch": nbytes,
            "design_bytes_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def end_to_end(ms_step: float, T: int, H: int, raw: bool) -> dict:
    """The whole fwd+bwd step on the method's own work and compulsory bytes."""
    th = float(T) * H
    flop = th * (FLOP_PER_TOKEN_HEAD["fwd"] + FLOP_PER_TOKEN_HEAD["bwd"])
    cb = COMPULSORY_BYTES_PER_TOKEN_HEAD[raw]
    nbytes = th * (cb["fwd"] + cb["bwd"])
    sec = ms_step * 1e-3
    return {"algorithmic_flop": flop, "tflops": round(flop / sec / 1e12, 2),
            "mfma_frac": round(flop / sec / 1e12 / PEAK_BF16_TFLOPS, 4),
            "compulsory_bytes": nbytes, "gbs": round(nbytes / sec / 1e9, 1),
            "hbm_frac": round(nbytes / sec / 1e9 / PEAK_HBM_GBS, 4)}


class HipEvents:
    """Per-kernel HIP event pairs recorded from the library's launch hook.
    The events are created beforehand (`reserve`): creating one can take long
    enough, on some hosts, for the launching thread to fall behind the GPU
    inside the timed region."""

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
        self.pool = []

    def _create(self):
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def reserve(self, n):
        self.pool.extend(self._create() for _ in range(n))

    def _event(self):
        return self.pool.pop() if self.pool else self._create()

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
        for e in self.pool:
            self.hip.hipEventDestroy(e)
        self.pool = []
        return out


class LaunchCounter:
    """Counts the library's launches (a hook that records nothing)."""

    def __init__(self):
        self.n = 0

    def hook(self, name, end, stream):
        self.n += 1


def fingerprint() -> str:
    """sha256 (16 hex digits) over the kernel sources; counter figures taken
    on other sources are stale."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if p.endswith((".hip", ".h", ".cpp")):
            h.update(os.path.basename(p).encode())
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def _short(kernel_name: str) -> str:
    for k in ("chunk_map", "seg_map", "fwd_prep", "fwd_scan", "fwd_out", "bwd_scan", "bwd_intra",
              "finalize", "zero_params", "walk", "conv_fwd", "conv_bwd", "conv_reduce", "conv_zero",
              "attn_fwd", "attn_delta", "attn_dq", "attn_dkdv", "rowmap_keys", "rowmap_tile_sort",
              "rowmap_merge", "rowmap_add"):
        if k + "_kernel" in kernel_name:
            return k
    return "copy" if "copyBuffer" in kernel_name else kernel_name[:40]


def _rocprof_rows(folder: str, query_db: str, csv_name: str):
    """Rows of a rocprofv3 output folder, from its SQLite results (the default
    output format) or its CSV files."""
    import sqlite3
    dbs = glob.glob(os.path.join(folder, "**", "*_results.db"), recursive=True)
    for f in dbs:
        con = sqlite3.connect(f)
        con.row_factory = sqlite3.Row
        yield from (dict(r) for r in con.execute(query_db))
        con.close()
    if not dbs:
        for f in glob.glob(os.path.join(folder, "**", csv_name), recursive=True):
            yield from csv.DictReader(open(f))


def pmc_summary(folder: str) -> dict:
    """Mean per dispatch of every counter in a rocprofv3 --pmc run:
    {kernel: {counter: (dispatches, mean, grid_size)}}."""
    acc = {}
    q = ("select kernel_name as Kernel_Name, counter_name as Counter_Name, "
         "value as Counter_Value, grid_size as Grid_Size from counters_collection")
    for r in _rocprof_rows(folder, q, "*counter_collection.csv"):
        key = (_short(r["Kernel_Name"]), r["Counter_Name"], int(r["Grid_Size"]))
        acc.setdefault(key, []).append(float(r["Counter_Value"]))
    if not acc:
        raise SystemExit(f"no counter records under {folder}")
    out = {}
    for (k, c, grid), v in sorted(acc.items()):
        out.setdefault(k, {})[c] = (len(v), statistics.fmean(v), grid)
    return out


def trace_summary(folder: str) -> dict:
    """Per-kernel dispatch count, total and mean duration (us) of a rocprofv3
    --kernel-trace run."""
    acc = {}
    q = "select name as Kernel_Name, start as Start_Timestamp, end as End_Timestamp from kernels"
    for r in _rocprof_rows(folder, q, "*kernel_trace.csv"):
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        acc.setdefault(_short(r["Kernel_Name"]), []).append(dur)
    if not acc:
        raise SystemExit(f"no kernel records under {folder}")
    return {k: (len(v), sum(v), statistics.fmean(v)) for k, v in acc.items()}


def profile_figures(workload: str, kernel: str, fp: str):
    """Counter figures recorded in profiles/ for this workload and kernel
    (a `figures:` JSON line in the summary), if taken on these sources."""
    for p in sorted(glob.glob(os.path.join(PROFILES, f"*{workload}*.md"))):
        for line in open(p):
            if line.startswith("figures: "):
                fig = json.loads(line[len("figures: "):])
                if fig.get("kernel") == kernel and fig.get("workload") == workload:
                    if fig.get("fingerprint") == fp:
                        return fig
    return None


def time_unit(torch, fn, samples=15, calls=20):
    """Median over `samples` of (HIP-event time of `calls` back-to-back calls) / calls."""
    out = []
    for _ in range(samples):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(calls):
            fn()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / calls)
    return statistics.median(out)


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
    4 heads per host thread of the same document(s), fwd + bwd."""
    import numpy as np
    from kda_chunked_amd import inputs as I
    from oracle import kda_oracle as ko
    nh = min(w.H, 4 * threads)
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


def make_runner(w, torch):
    """Device inputs and output buffers of workload w, and closures that run
    one fwd (saving or not), one bwd (saved or replay), one step and one
    replay pair on the current stream."""
    from kda_chunked_amd.binding import KDA
    inp, dev = make_device_inputs(w, torch)
    kda = KDA(w.T, w.H, len(w.doc_lens), gate=w.gate, l2norm=w.l2norm)
    A_log, dt_bias = dev.get("A_log"), dev.get("dt_bias")
    grads = dict(dq=torch.empty_like(dev["q"]), dk=torch.empty_like(dev["k"]),
                 dv=torch.empty_like(dev["v"]), dbeta=torch.empty_like(dev["beta"]),
                 dgate=torch.empty_like(dev["gate"]))
    if w.gate == "raw":
        grads.update(dA_log=torch.empty_like(A_log), ddt_bias=torch.empty_like(dt_bias))
    o = torch.empty_like(dev["v"])
    args_in = (dev["q"], dev["k"], dev["v"], dev["beta"], dev["gate"], dev["cu"])

    def fwd(save=True):
        kda.forward(*args_in, A_log, dt_bias, save=save, o=o)

    def bwd(replay=False):
        kda.backward(*args_in, dev["dO"], A_log, dt_bias, replay=replay, out=grads)

    def step():
        fwd()
        bwd()

    def replay_pair():
        fwd(save=False)
        bwd(replay=True)

    return inp, {"fwd": fwd, "bwd": bwd, "step": step, "replay_pair": replay_pair,
                 "kda": kda, "dev": dev, "grads": grads, "o": o}


# The other rows of the deterministic package's timing table that this
# repository's workloads reproduce (flashinfer PR #8909, timing tables): timed
# with the pages' protocol outside the timed region, as extra keys.
SECONDARY_ROWS = (("4doc", False), ("4doc", True), ("R2", False), ("m2", False), ("1doc", False))


def time_row(w, replay, torch) -> dict:
    """fwd, bwd and fwd+bwd ms (median of 15 samples of 20 back-to-back calls)
    of one row; replay rows time the pair fwd(no save) + bwd(replay)."""
    _, run = make_runner(w, torch)
    for _ in range(3):
        (run["replay_pair"] if replay else run["step"])()
    torch.cuda.synchronize()
    key = f"{w.key}:{'replay' if replay else 'saved'}"
    if replay:
        out = {"fwd_ms": time_unit(torch, lambda: run["fwd"](save=False)),
               "bwd_ms": time_unit(torch, lambda: run["bwd"](replay=True)),
               "fwd_bwd_ms": time_unit(torch, run["replay_pair"])}
    else:
        out = {"fwd_ms": time_unit(torch, run["fwd"]), "bwd_ms": time_unit(torch, run["bwd"]),
               "fwd_bwd_ms": time_unit(torch, run["step"])}
    out = {k: round(v, 4) for k, v in out.items()}
    out["tokens_per_s"] = round(w.T / (out["fwd_bwd_ms"] * 1e-3), 1)
    page = PAGE_FWD_BWD_MS.get(w.key + (":replay" if replay else ""))
    out["page_gb300_fwd_bwd_ms"] = page
    del run
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    print(f"[bench] row {key}: {out}", file=sys.stderr, flush=True)
    return {key: out}


def time_conv(torch) -> dict:
    """The width-4 causal conv1d + SiLU op on the 4doc layout (16384 tokens,
    the q, k, v channels of 64 heads x 128 = 24576, halo on): fwd and bwd ms
    with the pages' protocol, against the HBM peak on its compulsory bytes
    (fwd reads x and writes y; bwd reads x and dy and writes dx; bf16)."""
    import numpy as np
    from kda_chunked_amd import inputs as I
    from kda_chunked_amd.binding import ConvSiLU
    w = I.CONV_BY_NAME["conv_4doc"]
    inp = I.make_conv_inputs(w)
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    x, dy, halo = bf(inp["x"]), bf(inp["dy"]), bf(inp["halo"])
    wt = torch.from_numpy(inp["w"]).cuda()
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    op = ConvSiLU(w.T, w.D, len(w.doc_lens), bias=w.bias, halo=w.halo)
    y = torch.empty_like(x)
    out = dict(dx=torch.empty_like(x), dw=torch.empty_like(wt), dhalo=torch.empty_like(halo))
    fwd = lambda: op.forward(x, wt, cu, None, halo, y=y)
    bwd = lambda: op.backward(x, wt, cu, dy, None, halo, out=out)
    for _ in range(3):
        fwd()
        bwd()
    torch.cuda.synchronize()
    f_ms, b_ms = time_unit(torch, fwd), time_unit(torch, bwd)
    n = float(w.T) * w.D
    fb, bb = 4.0 * n, 6.0 * n
    res = {"workload": f"conv_4doc: {w.T} tokens x {w.D} channels, width 4, halo",
           "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
           "fwd": {"bound": "hbm", "achieved": round(fb / (f_ms * 1e-3) / 1e9, 1),
                   "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": round(fb / (f_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
           "bwd": {"bound": "hbm", "achieved": round(bb / (b_ms * 1e-3) / 1e9, 1),
                   "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": round(bb / (b_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}}
    print(f"[bench] conv: {res}", file=sys.stderr, flush=True)
    return res


PAGE_ATTN_STEP_MS = 4.527      # flashinfer PR #7774, GB200 table: zz_cp1_r0_16461 (Cake)


def time_attn(torch) -> dict:
    """Packed-varlen causal GQA attention (head dim 256) on the 16461-query,
    24693-key, 8-segment layout with 24 query and 4 key heads: forward,
    backward (bf16 dk, dv) and the pages' training step of one layer under
    activation checkpointing (2 x forward + backward), median of HIP-event
    timings, against the bf16 MFMA peak on the algorithmic FLOP (4 D per
    visible (query, key) pair and query head forward, 10 D backward)."""
    import numpy as np
    from kda_chunked_amd import inputs as I
    from kda_chunked_amd.binding import ATTN_DKV_BF16, GQAAttention
    w = I.ATTN_BY_NAME["attn_cp1_16461"]
    inp = I.make_attn_inputs(w)
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v, dO = bf(inp["q"]), bf(inp["k"]), bf(inp["v"]), bf(inp["dO"])
    cq, ck = torch.from_numpy(inp["cu_q"]).cuda(), torch.from_numpy(inp["cu_k"]).cuda()
    op = GQAAttention(w.Tq, w.Tk, len(w.q_lens), w.Hq, w.Hkv)
    o, lse = op.forward(q, k, v, cq, ck)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fwd = lambda: op.forward(q, k, v, cq, ck, o=o, lse=lse)
    bwd = lambda: op.backward(q, k, v, cq, ck, o, lse, dO, ATTN_DKV_BF16, dk=dk, dv=dv, dq=dq)

    def step():
        fwd()
        fwd()
        bwd()
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    f_ms = time_unit(torch, fwd, samples=7, calls=5)
    b_ms = time_unit(torch, bwd, samples=7, calls=3)
    s_ms = time_unit(torch, step, samples=5, calls=2)
    pairs = float(w.visible_pairs()) * w.Hq
    ff, bf_ = 4.0 * w.D * pairs, 10.0 * w.D * pairs
    rate = lambda fl, ms: round(fl / (ms * 1e-3) / 1e12, 1)
    res = {"workload": (f"attn_cp1_16461: Tq {w.Tq}, Tk {w.Tk}, {len(w.q_lens)} segments, "
                        f"Hq {w.Hq}, Hkv {w.Hkv}, D {w.D}, bottom-right causal"),
           "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4), "step_ms": round(s_ms, 4),
           "page_gb200_step_ms": PAGE_ATTN_STEP_MS,
           "fwd": {"bound": "mfma", "achieved": rate(ff, f_ms), "peak": PEAK_BF16_TFLOPS,
                   "unit": "TFLOP/s", "frac": round(ff / (f_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
           "bwd": {"bound": "mfma", "achieved": rate(bf_, b_ms), "peak": PEAK_BF16_TFLOPS,
                   "unit": "TFLOP/s",
                   "frac": round(bf_ / (b_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}}
    print(f"[bench] attn: {res}", file=sys.stderr, flush=True)
    return res


def time_cp(torch, ranks=4) -> dict:
    """One rank's share of the 1doc sequence split contiguously over `ranks`
    ranks (the last rank: its fragment continues the document), with the
    exchange between ranks left out: the state summary (prep kept in the
    saved set), ranks - 1 transfer steps, the forward from the walked state,
    the gradient summary, ranks - 1 transposed transfer steps and the
    backward; against the plain forward + backward of the same fragment."""
    import numpy as np
    from kda_chunked_amd import inputs as I
    from kda_chunked_amd.binding import KDA, kda_state_apply
    w = I.BY_NAME["1doc"]
    inp = I.make_inputs(w)
    T = w.T // ranks
    a0 = w.T - T
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x[a0:]).view(np.int16)).view(
        torch.bfloat16).cuda()
    q, k, v, beta, dO = (bf(inp[n]) for n in ("q", "k", "v", "beta", "dO"))
    g = torch.from_numpy(np.ascontiguousarray(inp["gate"][a0:])).cuda()
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    kda = KDA(T, w.H, 1, gate=w.gate, l2norm=w.l2norm)
    args = (q, k, v, beta, g, cu)
    st = lambda: torch.zeros(w.H, 128, 128, dtype=torch.float32, device="cuda")
    S_init, s_fin, dS, ds_in, y = st(), st(), st(), st(), st()
    o = torch.empty_like(v)
    M, B = kda.state_summary(*args, keep_prep=True)
    kda.forward(*args, o=o, s_init=S_init, s_final=s_fin, prep_done=True)
    grads = kda.backward(*args, dO, s_init=S_init, ds_final=dS, ds_init=ds_in)

    def share():
        kda.state_summary(*args, keep_prep=True)
        for _ in range(ranks - 1):
            kda_state_apply(M, S_init, B, y=y)
        kda.forward(*args, o=o, s_init=S_init, s_final=s_fin, prep_done=True)
        kda.state_grad_summary(*args, dO)
        for _ in range(ranks - 1):
            kda_state_apply(M, dS, B, transpose=True, y=y)
        kda.backward(*args, dO, s_init=S_init, ds_final=dS, ds_init=ds_in, out=grads)

    def plain():
        kda.forward(*args, o=o)
        kda.backward(*args, dO, out=grads)
    for _ in range(2):
        share()
        plain()
    torch.cuda.synchronize()
    parts = {
        "summary_ms": lambda: kda.state_summary(*args, keep_prep=True),
        "apply_ms": lambda: kda_state_apply(M, S_init, B, y=y),
        "fwd_state_ms": lambda: kda.forward(*args, o=o, s_init=S_init, s_final=s_fin,
                                            prep_done=True),
        "grad_summary_ms": lambda: kda.state_grad_summary(*args, dO),
        "bwd_state_ms": lambda: kda.backward(*args, dO, s_init=S_init, ds_final=dS,
                                             ds_init=ds_in, out=grads),
    }
    res = {"workload": (f"1doc split over {ranks} ranks, last rank's share: {T} tokens x "
                        f"{w.H} heads, one continuing document, gate {w.gate}, "
                        f"L2 {'fused' if w.l2norm else 'off'}")}
    for name, fn in parts.items():
        res[name] = round(time_unit(torch, fn, samples=7, calls=5), 4)
    res["share_step_ms"] = round(time_unit(torch, share, samples=7, calls=3), 4)
    res["plain_step_ms"] = round(time_unit(torch, plain, samples=7, calls=3), 4)
    res["overhead"] = round(res["share_step_ms"] / res["plain_step_ms"], 3)
    res["share_tokens_per_s"] = round(T / (res["share_step_ms"] * 1e-3), 1)
    print(f"[bench] cp: {res}", file=sys.stderr, flush=True)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="1doc")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-units", action="store_true",
                    help="skip the fwd / bwd / replay unit timings")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the other workloads' rows (4doc saved and replay, R2, m2)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after the steps, copy MIB MiB device to device once (a plain copy "
                         "kernel of known size, for scaling HBM byte counters)")
    ap.add_argument("--pmc-summary", metavar="DIR", help="tabulate a rocprofv3 --pmc run and exit")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="tabulate a rocprofv3 --kernel-trace run and exit")
    ap.add_argument("--fingerprint", action="store_true", help="print the source hash and exit")
    ap.add_argument("--leg", choices=("kda", "conv", "attn", "cp"), default="kda",
                    help="time only the conv1d + SiLU leg, the attention leg, or one rank's "
                         "share of a sequence split over ranks (for profiling runs)")
    args = ap.parse_args()
    if args.fingerprint:
        print(fingerprint())
        return
    if args.trace_summary:
        summ = trace_summary(args.trace_summary)
        tot = sum(v[1] for v in summ.values())
        print("| kernel | dispatches | total us | mean us | % |")
        print("|---|---:|---:|---:|---:|")
        for k, (n, t, m) in sorted(summ.items(), key=lambda kv: -kv[1][1]):
            print(f"| {k} | {n} | {t:.1f} | {m:.1f} | {100 * t / tot:.1f} |")
        return
    if args.pmc_summary:
        summ = pmc_summary(args.pmc_summary)
        print("| kernel | counter | dispatches | mean per dispatch | grid |")
        print("|---|---|---:|---:|---:|")
        for k, cs in summ.items():
            for c, (n, m, grid) in cs.items():
                print(f"| {k} | {c} | {n} | {m:.6g} | {grid} |")
        return
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this build runs on one GPU "
              "(heads or sequence shards would split across GPUs; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from kda_chunked_amd import inputs as I
    from kda_chunked_amd.binding import lib, set_launch_hook

    lib()
    if args.leg != "kda":
        if args.calibrate_copy:
            src = torch.ones(args.calibrate_copy << 20, dtype=torch.uint8, device="cuda")
            torch.empty_like(src).copy_(src)
            torch.cuda.synchronize()
        legs = {"conv": time_conv, "attn": time_attn, "cp": time_cp}
        print(json.dumps(legs[args.leg](torch)), flush=True)
        return
    w = I.BY_NAME[args.workload]
    inp, run = make_runner(w, torch)
    step, fwd, bwd, replay_pair = run["step"], run["fwd"], run["bwd"], run["replay_pair"]

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, per-kernel HIP events from the hook
    counter = LaunchCounter()
    set_launch_hook(counter.hook)
    step()
    set_launch_hook(None)
    torch.cuda.synchronize()
    ev = HipEvents()
    ev.reserve(counter.n * args.steps + 16)
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

    units = {}
    if not args.no_units:
        units["fwd_ms"] = time_unit(torch, fwd)
        units["bwd_ms"] = time_unit(torch, bwd)
        units["fwd_bwd_ms"] = time_unit(torch, step)
        units["replay_fwd_bwd_ms"] = time_unit(torch, replay_pair)
        units = {k: round(v, 4) for k, v in units.items()}

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    chunk_heads = w.T * w.H / 64.0    # chunk-head equivalents per launch
    raw = w.gate == "raw"
    per_kernel = {k: kernel_roofline(k, kern_avg[k], chunk_heads, raw)
                  for k in kern_avg if k in MAC_PER_CHUNK_HEAD}
    # the dominant contraction kernel: the longest MFMA kernel of the step
    dom = max((k for k in per_kernel if k in MFMA_KERNELS), key=lambda k: kern_avg[k])
    fp = fingerprint()
    fig = profile_figures(w.name, dom, fp)
    r = per_kernel[dom]
    sec = kern_avg[dom] * 1e-3
    comp = float(BWD_INTRA_COMPULSORY_BYTES_PER_TOKEN_HEAD[raw]) * w.T * w.H \
        if dom == "bwd_intra" else None
    traffic = fig["traffic_bytes"] if fig else None
    roofline = {"bound": "mfma", "kernel": dom, "achieved": r["achieved"], "peak": r["peak"],
                "unit": r["unit"], "frac": r["frac"], "traffic": traffic,
                "algorithmic_flop_per_launch": r["algorithmic_flop_per_launch"],
                "avg_launch_ms": round(kern_avg[dom], 4)}
    if comp is not None:
        roofline["compulsory_bytes_per_launch"] = comp
        roofline["compulsory_hbm_frac"] = round(comp / sec / 1e9 / PEAK_HBM_GBS, 4)
        roofline["traffic_over_compulsory"] = round(traffic / comp, 3) if traffic else None
    if fig:
        roofline["mfma_busy_pct"] = fig.get("mfma_busy_pct")
        roofline["executed_mfma_tflops"] = round(
            fig["mfma_flop"] / sec / 1e12, 2) if "mfma_flop" in fig else None

    rows = {}
    conv = attn = cp = None
    if not args.no_rows:
        for name, replay in SECONDARY_ROWS:
            if name == w.name:
                continue
            rows.update(time_row(I.BY_NAME[name], replay, torch))
        conv = time_conv(torch)
        attn = time_attn(torch)
        cp = time_cp(torch)

    line = {
        "metric": METRIC,
        "value": round(w.T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(w.T / (ms_step * 1e-3) / (w.T / (PAGE_FWD_BWD_MS[w.key] * 1e-3)), 4)
                        if w.key in PAGE_FWD_BWD_MS else None),
        "vs_baseline_note": ("ratio to the GB300 fwd+bwd figure of this row on flashinfer PR "
                             "#8909 (other hardware, context only)"),
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.key + ":saved", "tokens": w.T, "heads": w.H, "head_dim": 128,
                   "docs": list(w.doc_lens), "chunk": 64},
        "roofline": roofline,
        "end_to_end": end_to_end(ms_step, w.T, w.H, raw),
        "token_heads_per_s": round(w.T * w.H / (ms_step * 1e-3), 1),
        "kernels_ms": {k: round(v, 4) for k, v in sorted(kern_avg.items())},
        "kernels_roofline": {k: {"bound": v["bound"], "frac": v["frac"],
                                 "design_bytes_frac": v["design_bytes_frac"]}
                             for k, v in sorted(per_kernel.items())},
        "wall_s_timed": round(wall, 3),
        "source_fingerprint": fp,
    }
    line.update(units)
    if rows:
        line["rows"] = rows
    if conv:
        line["conv1d_silu"] = conv
    if attn:
        line["gqa_attention"] = attn
    if cp:
        line["kda_cp_rank_share"] = cp
    if not args.no_cpu:
        from oracle import kda_oracle as ko
        line["cpu_baseline"] = cpu_baseline(w, inp, ko.default_threads())
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
