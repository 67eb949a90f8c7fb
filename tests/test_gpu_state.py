"""One rank's share of a packed sequence split over ranks, run on one GPU
(flashinfer PR #7176, opening section: the recurrent state crosses fragment
boundaries as FP32 affine summaries S_out = M S_in + B, and its gradient as
dS_in = M^T dS_out + B'). Each case cuts a workload into fragments, runs them
one after another through the boundary-state entry points exactly as ranks
would (state maps and zero-entry runs first, the transfer walk over the
summaries, then the final runs), and compares the stitched outputs and
gradients with the FP64 oracle on the unsplit sequence; every fragment's
leaving state and entering-state gradient is checked against the oracle run
on that fragment with the same boundary states, and the state map against
the oracle's (s_final from s_init = I with V = 0)."""

import numpy as np
import pytest
import torch

from gpu_common import TOL, f64, gpu_grads_f64, rel_l2, run_gpu, run_oracle, to_device
from kda_chunked_amd import inputs as I

pytestmark = pytest.mark.gpu

HD = 128
# relative L2 bound of fp32 states carried over a fragment (same budget as o)
TOL_STATE = 2e-3
# relative L2 bound of the state map M of a fragment of n chunks: each chunk
# step's correction -Ke^T Tb Kd S takes the state and the decayed keys Kd
# rounded to bf16 (unit roundoff u = 2^-8, relative RMS at most u / sqrt(3)
# each), as in the forward; the roundings of different steps are independent,
# so over n steps they add in quadrature
def tol_map(n):
    return 2.0 ** -8 * np.sqrt(2 * n / 3)


# fp32 holds no entry below 2^-126, and an M of norm below 2^-100 moves no
# state of ordinary size: errors of M are measured against this floor
M_FLOOR = 2.0 ** -100
# bound relative to the unsplit run for per-token outputs: the split changes
# only where chunks start and what the boundary states carry
SPLIT_SLACK = (1.05, 1e-4)
# slow decay keeps the state large across hundreds of tokens, and its bf16
# rounding in the forward's V - Kd S product weighs more beside the output's
# own rounding: the unsplit library sits at about 1.1 x the default bound there
SLOW_FACTOR = 1.25


def fragments(inp, cuts):
    """Slices [a, b) of the packed inputs at the token cuts; each slice's
    cu_seqlens starts a new document at 0 and ends at its length. Returns
    (slices, cont) with cont[r] true when fragment r continues a document."""
    cu = inp["cu_seqlens"].astype(np.int64)
    T = int(cu[-1])
    edges = [0] + list(cuts) + [T]
    out, cont = [], []
    for a, b in zip(edges[:-1], edges[1:]):
        f = {}
        for key in ("q", "k", "v", "beta", "gate", "dO"):
            f[key] = np.ascontiguousarray(inp[key][a:b])
        for key in ("A_log", "dt_bias"):
            if key in inp:
                f[key] = inp[key]
        inner = cu[(cu > a) & (cu < b)] - a
        f["cu_seqlens"] = np.concatenate([[0], inner, [b - a]]).astype(np.int32)
        out.append(f)
        cont.append(a > 0 and a not in cu)
    return out, cont


def run_split(w, inp, cuts):
    """The ranks' protocol, fragment by fragment on one GPU; also the zero-entry
    runs that the summaries stand for (o_zero, s_zero, ds_zero)."""
    from kda_chunked_amd.binding import KDA, kda_state_apply
    frags, cont = fragments(inp, cuts)
    R = len(frags)
    devs = [to_device(f) for f in frags]
    kdas = [KDA(int(f["cu_seqlens"][-1]), w.H, len(f["cu_seqlens"]) - 1, gate=w.gate,
                l2norm=w.l2norm) for f in frags]
    st = lambda: torch.zeros(w.H, HD, HD, dtype=torch.float32, device="cuda")
    args = lambda d: (d["q"], d["k"], d["v"], d["beta"], d["gate"], d["cu_seqlens"])
    par = lambda d: (d.get("A_log"), d.get("dt_bias"))
    # forward summaries (the prep kept in each saved set), then the transfer
    # walk over the gathered (M, B)
    MB = [kdas[r].state_summary(*args(devs[r]), *par(devs[r]), keep_prep=True)
          for r in range(R)]
    M = [m for m, _ in MB]
    S_init = [st()]
    for r in range(1, R):
        S_init.append(kda_state_apply(M[r - 1], S_init[r - 1], MB[r - 1][1]) if cont[r] else st())
    # forward from the walked states, on the kept prep, saving
    o, s_final = [], []
    for r in range(R):
        s_final.append(st())
        o.append(kdas[r].forward(*args(devs[r]), *par(devs[r]), s_init=S_init[r],
                                 s_final=s_final[r], prep_done=True))
    # backward summaries from the saved sets, the reverse walk, the backward
    Bb = [kdas[r].state_grad_summary(*args(devs[r]), devs[r]["dO"], *par(devs[r]))
          for r in range(R)]
    dS_final = [None] * R
    dS_final[R - 1] = st()
    for r in range(R - 2, -1, -1):
        dS_final[r] = (kda_state_apply(M[r + 1], dS_final[r + 1], Bb[r + 1], transpose=True)
                       if cont[r + 1] else st())
    grads, ds_init = [], []
    for r in range(R):
        ds_init.append(st())
        grads.append(kdas[r].backward(*args(devs[r]), devs[r]["dO"], *par(devs[r]),
                                      s_init=S_init[r], ds_final=dS_final[r], ds_init=ds_init[r]))
    torch.cuda.synchronize()
    # what the summaries stand for: zero-entry forward and zero-exit backward
    # (replay, so the saved sets above stay as they are)
    o_zero, s_zero, ds_zero = [], [], []
    for r in range(R):
        s_zero.append(st())
        o_zero.append(kdas[r].forward(*args(devs[r]), *par(devs[r]), save=False,
                                      s_final=s_zero[r]))
        ds_zero.append(st())
        kdas[r].backward(*args(devs[r]), devs[r]["dO"], *par(devs[r]), replay=True,
                         s_init=S_init[r], ds_init=ds_zero[r])
    torch.cuda.synchronize()
    return dict(frags=frags, cont=cont, M=M, B=[b for _, b in MB], Bb=Bb, S_init=S_init,
                s_final=s_final, o=o, o_zero=o_zero, s_zero=s_zero, ds_zero=ds_zero,
                dS_final=dS_final, ds_init=ds_init, grads=grads, kdas=kdas, devs=devs)


def stitch(w, res):
    o = np.concatenate([f64(x) for x in res["o"]])
    gs = [gpu_grads_f64(w, g) for g in res["grads"]]
    out = {}
    for key in gs[0]:
        if key in ("dA_log", "ddt_bias"):
            out[key] = sum(g[key] for g in gs)
        else:
            out[key] = np.concatenate([g[key] for g in gs])
    return o, out


def oracle_fragment(w, frag, s_init, ds_final):
    from oracle import kda_oracle as ko
    f = I.as_f64(frag)
    args = (f["cu_seqlens"], f["q"], f["k"], f["v"], f["beta"], f["gate"])
    extra = dict(A_log=f["A_log"], dt_bias=f["dt_bias"]) if w.gate == "raw" else {}
    _, s_fin = ko.fwd(*args, gate_form=w.gate, l2norm=w.l2norm, s_init=s_init,
                      final_state=True, **extra)
    g = ko.bwd(*args, f["dO"], gate_form=w.gate, l2norm=w.l2norm, s_init=s_init,
               ds_final=ds_final, **extra)
    return s_fin, g["ds_init"]


SLOW = (-8.0, -6.0)   # A_log range of slow decay: M stays far from zero over a fragment
CASES = [
    # (docs, H, gate, l2, cuts, A_log range): cuts inside documents, at a
    # document start, off the 64-token chunk grid, and a fragment holding
    # several documents
    ((700, 300, 520), 4, "g", False, (250, 700, 1100), None),
    ((900, 411), 3, "raw", False, (333, 901), None),
    ((1000, 200), 2, "g", True, (130, 640), None),
    ((1500, 300), 2, "raw", False, (400, 1000, 1600), SLOW),
    # few chains: the fragments' scans run segmented (segments of 16 chunks)
    ((5200,), 1, "g", False, (1100, 3000), None),
    ((4100, 900), 2, "raw", False, (2500,), None),
    ((4000,), 1, "raw", True, (1700,), SLOW),
]
IDS = ["g-3doc-H4", "raw-2doc-H3", "g-l2-2doc-H2", "raw-slow-2doc-H2", "g-seg-1doc-H1",
       "raw-seg-2doc-H2", "raw-slow-seg-l2-1doc-H1"]


def workload(docs, H, gate, l2, alog, seed, name):
    kw = {} if alog is None else dict(alog_range=alog)
    return I.custom(docs, H, gate=gate, l2norm=l2, seed=seed, name=name, **kw)


@pytest.mark.parametrize("docs,H,gate,l2,cuts,alog", CASES, ids=IDS)
def test_split_matches_unsplit_oracle(docs, H, gate, l2, cuts, alog):
    w = workload(docs, H, gate, l2, alog, 61, "split")
    print(f"[case] split {w.key} docs={w.doc_lens} H={H} cuts={cuts}", flush=True)
    inp = I.make_inputs(w)
    res = run_split(w, inp, cuts)
    o, gg = stitch(w, res)
    oref, gref = run_oracle(w, inp)
    errs = {"o": rel_l2(o, oref)}
    errs.update({k: rel_l2(gg[k], v) for k, v in gref.items()})
    print("[parity] split " + ", ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)
    uo, ug, _ = run_gpu(w, to_device(inp))
    ugg = gpu_grads_f64(w, ug)
    uerrs = {"o": rel_l2(f64(uo), oref)}
    uerrs.update({k: rel_l2(ugg[k], v) for k, v in gref.items()})
    print("[parity] unsplit " + ", ".join(f"{k}={v:.3e}" for k, v in uerrs.items()), flush=True)
    bar = {k: TOL[k] * (SLOW_FACTOR if alog == SLOW else 1.0) for k in errs}
    bad = {k: v for k, v in errs.items() if not v <= bar[k]}
    bad.update({"unsplit " + k: v for k, v in uerrs.items() if not v <= bar[k]})
    a, b = SPLIT_SLACK
    bad.update({"vs unsplit " + k: (v, uerrs[k]) for k, v in errs.items()
                if k not in ("dA_log", "ddt_bias") and not v <= a * uerrs[k] + b})
    assert not bad, bad
    if alog is not None:
        # slow decay: without the handed-over states the outputs miss the bar
        e0 = rel_l2(np.concatenate([f64(x) for x in res["o_zero"]]), oref)
        print(f"[control] split without the handover: o={e0:.3e}", flush=True)
        assert e0 > 10 * TOL["o"], e0
    # each fragment's boundary states against the oracle on that fragment, fed
    # the same entering state and leaving gradient; the summaries B and B'
    # against the oracle from a zero entering state and leaving gradient, and
    # against the library's own zero-entry runs
    for r, frag in enumerate(res["frags"]):
        s_ref, ds_ref = oracle_fragment(w, frag, f64(res["S_init"][r]), f64(res["dS_final"][r]))
        b_ref, bb_ref = oracle_fragment(w, frag, None, np.zeros((w.H, HD, HD)))
        e = dict(s_final=rel_l2(f64(res["s_final"][r]), s_ref),
                 ds_init=rel_l2(f64(res["ds_init"][r]), ds_ref),
                 B=rel_l2(f64(res["B"][r]), b_ref), Bb=rel_l2(f64(res["Bb"][r]), bb_ref),
                 B_vs_run=rel_l2(f64(res["B"][r]), f64(res["s_zero"][r])),
                 Bb_vs_run=rel_l2(f64(res["Bb"][r]), f64(res["ds_zero"][r])))
        print(f"[parity] fragment {r}: " + ", ".join(f"{k}={v:.3e}" for k, v in e.items()),
              flush=True)
        bad = {k: v for k, v in e.items() if not v <= TOL_STATE}
        assert not bad, (r, bad)


MAP_CASES = [0, 3, 4, 6]


@pytest.mark.parametrize("docs,H,gate,l2,cuts,alog", [CASES[i] for i in MAP_CASES],
                         ids=[IDS[i] for i in MAP_CASES])
def test_state_map_matches_oracle(docs, H, gate, l2, cuts, alog):
    """M of a single-document fragment is the oracle's s_final from s_init = I
    with V = 0; a fragment of several documents maps to zero, an empty one to
    the identity (with B = 0 and a zero gradient summary)."""
    from kda_chunked_amd.binding import KDA
    from oracle import kda_oracle as ko
    w = workload(docs, H, gate, l2, alog, 62, "map")
    inp = I.make_inputs(w)
    frags, _ = fragments(inp, cuts)
    eye = np.broadcast_to(np.eye(HD), (H, HD, HD)).copy()
    errs, bars = {}, {}
    for r, frag in enumerate(frags):
        n_chunks = (len(frag["q"]) + 63) // 64
        d = to_device(frag)
        n = len(frag["cu_seqlens"]) - 1
        kda = KDA(int(frag["cu_seqlens"][-1]), H, n, gate=gate, l2norm=l2)
        M, _ = kda.state_summary(d["q"], d["k"], d["v"], d["beta"], d["gate"], d["cu_seqlens"],
                                 d.get("A_log"), d.get("dt_bias"), want_B=False)
        M = f64(M)
        if n > 1:
            assert not M.any(), r
            continue
        f = I.as_f64(frag)
        # V = 0 leaves B = 0: s_final at s_init = I is M itself (a difference
        # of two runs would lose M, which decays far below B, to rounding)
        a = (f["cu_seqlens"], f["q"], f["k"], np.zeros_like(f["v"]), f["beta"], f["gate"])
        extra = dict(A_log=f["A_log"], dt_bias=f["dt_bias"]) if gate == "raw" else {}
        _, Mref = ko.fwd(*a, gate_form=gate, l2norm=l2, s_init=eye, final_state=True, **extra)
        errs[r] = np.linalg.norm(M - Mref) / max(np.linalg.norm(Mref), M_FLOOR)
        bars[r] = tol_map(n_chunks)
        print(f"[parity] state map fragment {r}: {errs[r]:.3e} |Mref|={np.linalg.norm(Mref):.3e} "
              f"chunks={n_chunks} bound={bars[r]:.3e}", flush=True)
    bad = {r: e for r, e in errs.items() if not e <= bars[r]}
    assert not bad, bad
    # an empty fragment: M = I, B = 0, B' = 0
    kda = KDA(0, H, 1, gate=gate, l2norm=l2)
    z = torch.zeros(0, H, HD, dtype=torch.bfloat16, device="cuda")
    zb = torch.zeros(0, H, dtype=torch.bfloat16, device="cuda")
    zg = (torch.zeros(0, H, HD, dtype=torch.float32, device="cuda") if gate == "g" else z)
    cu0 = torch.zeros(2, dtype=torch.int32, device="cuda")
    M0, B0 = kda.state_summary(z, z, z, zb, zg, cu0)
    dB0 = kda.state_grad_summary(z, z, z, zb, zg, cu0, z)
    assert torch.equal(M0.cpu(), torch.eye(HD).expand(H, HD, HD)), "empty fragment"
    assert not B0.any() and not dB0.any(), "empty fragment"


def test_boundary_states_are_reproducible_and_replay_equal():
    """Run the protocol twice: bitwise equal; the replay backward (forward
    recomputed from s_init) equals the saved one bitwise, and so do the
    gradient summary with its operand panels rebuilt and a forward that runs
    its own prep."""
    docs, H, gate, l2, cuts, alog = CASES[6]
    w = workload(docs, H, gate, l2, alog, 63, "rep")
    inp = I.make_inputs(w)
    a = run_split(w, inp, cuts)
    b = run_split(w, inp, cuts)
    for key in ("o", "s_final", "ds_init", "S_init", "dS_final", "M", "B", "Bb"):
        for x, y in zip(a[key], b[key]):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), key
    for ga, gb in zip(a["grads"], b["grads"]):
        for key, v in ga.items():
            if v is not None:
                assert torch.equal(v.view(torch.uint8), gb[key].view(torch.uint8)), key
    for r in range(len(a["frags"])):
        d = a["devs"][r]
        sf = torch.zeros(H, HD, HD, dtype=torch.float32, device="cuda")
        o = a["kdas"][r].forward(d["q"], d["k"], d["v"], d["beta"], d["gate"], d["cu_seqlens"],
                                 d.get("A_log"), d.get("dt_bias"), save=False,
                                 s_init=a["S_init"][r], s_final=sf)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.uint8), a["o"][r].view(torch.uint8)), r
        assert torch.equal(sf.view(torch.uint8), a["s_final"][r].view(torch.uint8)), r
        ds = torch.zeros(H, HD, HD, dtype=torch.float32, device="cuda")
        g = a["kdas"][r].backward(d["q"], d["k"], d["v"], d["beta"], d["gate"],
                                  d["cu_seqlens"], d["dO"], d.get("A_log"), d.get("dt_bias"),
                                  replay=True, s_init=a["S_init"][r],
                                  ds_final=a["dS_final"][r], ds_init=ds)
        dB = a["kdas"][r].state_grad_summary(d["q"], d["k"], d["v"], d["beta"], d["gate"],
                                             d["cu_seqlens"], d["dO"], d.get("A_log"),
                                             d.get("dt_bias"), replay=True)
        torch.cuda.synchronize()
        assert torch.equal(ds.view(torch.uint8), a["ds_init"][r].view(torch.uint8)), r
        assert torch.equal(dB.view(torch.uint8), a["Bb"][r].view(torch.uint8)), r
        for key, v in a["grads"][r].items():
            if v is not None and key != "ds_init":
                assert torch.equal(v.view(torch.uint8), g[key].view(torch.uint8)), (r, key)


@pytest.mark.parametrize("H", [1, 5])
def test_state_apply_matches_numpy(H):
    from kda_chunked_amd.binding import kda_state_apply
    rng = np.random.default_rng(64 + H)
    M = rng.standard_normal((H, HD, HD)).astype(np.float32) / 8
    x = rng.standard_normal((H, HD, HD)).astype(np.float32)
    B = rng.standard_normal((H, HD, HD)).astype(np.float32)
    t = lambda a: torch.from_numpy(a).cuda()
    for trans in (False, True):
        Mt = np.swapaxes(M, 1, 2) if trans else M
        ref = Mt.astype(np.float64) @ x.astype(np.float64) + B
        y = f64(kda_state_apply(t(M), t(x), t(B), transpose=trans))
        assert rel_l2(y, ref) <= 1e-5, trans
        y0 = f64(kda_state_apply(t(M), t(x), None, transpose=trans))
        assert rel_l2(y0, ref - B) <= 1e-5, trans
        # in place over x
        xx = t(x)
        kda_state_apply(t(M), xx, t(B), transpose=trans, y=xx)
        torch.cuda.synchronize()
        assert rel_l2(f64(xx), ref) <= 1e-5, trans
