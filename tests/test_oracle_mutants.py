"""Planted mistakes: every plausible slip in the oracle must fail a pin.

Each case copies ``oracle/kda_oracle.cpp`` into a temporary directory, plants
one mistake (a flipped sign, a dropped factor, a wrong operand or index),
compiles it, and runs a battery of the pins from ``test_oracle_pins.py``
(closed forms, finite differences, chunked-form agreement, invariants)
against the mutant. The test passes only if the battery rejects it. This runs
on the CPU only; the oracle in the repository is never modified.
"""

import concurrent.futures as cf
import os
import tempfile

import numpy as np
import pytest

from helpers import rel_l2, tiny_problem
from models import kda_chunked_fp64 as chunked
from oracle import kda_oracle as ko

SRC = os.path.join(os.path.dirname(ko.__file__), "kda_oracle.cpp")

MUTANTS = {
    "u_sign": ("ut[j] = vt[j] - acc;", "ut[j] = vt[j] + acc;"),
    "drop_beta_update": ("S[c * V + j] += b * kt[c] * ut[j];", "S[c * V + j] += kt[c] * ut[j];"),
    "drop_scale_fwd": ("ot[j] = P.scale * acc;", "ot[j] = acc;"),
    "decay_exponent": ("tk.a[i * K + c] = std::exp(g);", "tk.a[i * K + c] = std::exp(2.0 * g);"),
    "key_index": ("for (int c = 0; c < K; ++c) acc += S[c * V + j] * kt[c];",
                  "for (int c = 0; c < K; ++c) acc += S[c * V + j] * kt[j % K];"),
    "l2_power": ("tk.rq[i] = 1.0 / std::sqrt(sq + P.l2_eps);", "tk.rq[i] = 1.0 / (sq + P.l2_eps);"),
    "raw_dt_sign": ("softplus(gs[c] + in.dt_bias[h * K + c])", "softplus(gs[c] - in.dt_bias[h * K + c])"),
    "dk_sign": ("dkh[i * K + c] -= acc;", "dkh[i * K + c] += acc;"),
    "du_drop_beta": ("du[j] = bt * acc;", "du[j] = acc;"),
    "dg_wrong_operand": ("acc += dSp[c * V + j] * Sp[c * V + j];", "acc += dS[c * V + j] * Sp[c * V + j];"),
    "dS_drop_decay": ("dS[c * V + j] = at[c] * dSp[c * V + j];", "dS[c * V + j] = dSp[c * V + j];"),
    "dS_drop_scale": ("dS[c * V + j] += P.scale * qt[c] * dOt[j];", "dS[c * V + j] += qt[c] * dOt[j];"),
    "dq_drop_scale": ("dqh[i * K + c] = P.scale * acc;", "dqh[i * K + c] = acc;"),
    "dbeta_drop_key": ("db += kt[c] * acc;", "db += acc;"),
    "dSp_sign": ("dSp[c * V + j] = dS[c * V + j] - kt[c] * du[j];",
                 "dSp[c * V + j] = dS[c * V + j] + kt[c] * du[j];"),
    "l2_bwd_projection": ("dq[c] = tk.rq[i] * (dqh[i * K + c] - tk.q[i * K + c] * pq);",
                          "dq[c] = tk.rq[i] * dqh[i * K + c];"),
    "l2_bwd_swapped": ("dk[c] = tk.rk[i] * (dkh[i * K + c] - tk.k[i * K + c] * pk);",
                       "dk[c] = tk.rk[i] * (dkh[i * K + c] - tk.k[i * K + c] * pq);"),
    "raw_bwd_sigmoid": ("const double dz = dg[i * K + c] * (-ea) * sigmoid(z);",
                        "const double dz = dg[i * K + c] * (-ea) * sigmoid(-z);"),
    "dAlog_drop_g": ("dAlog += dg[i * K + c] * tk.g[i * K + c];", "dAlog += dg[i * K + c];"),
    "softplus_large_drop_x": ("if (x > 30.0) return x + std::log1p(std::exp(-x));",
                              "if (x > 30.0) return std::log1p(std::exp(-x));"),
    "softplus_large_sign": ("if (x > 30.0) return x + std::log1p(std::exp(-x));",
                            "if (x > 30.0) return -x + std::log1p(std::exp(-x));"),
    # boundary states of a split sequence
    "s_init_dropped_bwd": ("    if (d == 0 && bd.s_init) std::memcpy(S.data()",
                           "    if (false && bd.s_init) std::memcpy(S.data()"),
    "s_final_wrong_doc": ("if (d == P.N - 1 && bd.s_final)", "if (d == 0 && bd.s_final)"),
    "ds_final_wrong_doc": ("if (d == P.N - 1 && bd.ds_final)", "if (d == 0 && bd.ds_final)"),
    "ds_init_before_decay": ("std::memcpy(bd.ds_init + (int64_t)h * K * V, dS.data()",
                             "std::memcpy(bd.ds_init + (int64_t)h * K * V, dSp.data()"),
}


def _run(lib, p, **kw):
    return ko.fwd(p["cu"], p["q"], p["k"], p["v"], p["beta"], p["gate"], p.get("A_log"),
                  p.get("dt_bias"), gate_form=p["gate_form"], l2norm=p["l2norm"], lib=lib,
                  threads=1, **kw)


def _grad(lib, p, **kw):
    return ko.bwd(p["cu"], p["q"], p["k"], p["v"], p["beta"], p["gate"], p["dO"],
                  p.get("A_log"), p.get("dt_bias"), gate_form=p["gate_form"],
                  l2norm=p["l2norm"], lib=lib, threads=1, **kw)


def _fd_ok(lib, p, tol=1e-6, h=1e-6):
    g = _grad(lib, p)
    names = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta",
             "gate": "da" if p["gate_form"] == "raw" else "dg"}
    if p["gate_form"] == "raw":
        names.update(A_log="dA_log", dt_bias="ddt_bias")
    for inp, out in names.items():
        x = p[inp].reshape(-1)
        fd = np.zeros_like(x)
        for i in range(x.size):
            old = x[i]
            x[i] = old + h
            lp = float(np.sum(_run(lib, p) * p["dO"]))
            x[i] = old - h
            lm = float(np.sum(_run(lib, p) * p["dO"]))
            x[i] = old
            fd[i] = (lp - lm) / (2 * h)
        if not rel_l2(g[out].reshape(-1), fd) < tol:
            return False
    return True


def battery(lib):
    """Returns the names of the pins the library fails."""
    failed = []
    rng = np.random.default_rng(123)
    # closed form: two tokens, each gate form / L2 mode
    for gate, l2 in (("g", False), ("raw", False), ("g", True)):
        p = tiny_problem(rng, [2], 1, 5, 3, gate=gate, l2norm=l2, decay=1.0)
        o = _run(lib, p)
        q, k, v, b = p["q"][:, 0], p["k"][:, 0], p["v"][:, 0], p["beta"][:, 0]
        if l2:
            q = q / np.sqrt(np.sum(q * q, -1, keepdims=True) + 1e-6)
            k = k / np.sqrt(np.sum(k * k, -1, keepdims=True) + 1e-6)
        g = p["gate"][:, 0]
        if gate == "raw":
            g = -np.exp(p["A_log"][0]) * np.logaddexp(0.0, g + p["dt_bias"][0])
        a = np.exp(g)
        s = 5 ** -0.5
        ka = a[1] * k[0]
        u2 = v[1] - b[0] * (k[1] @ ka) * v[0]
        o1 = s * b[0] * (q[0] @ k[0]) * v[0]
        o2 = s * (b[0] * (q[1] @ ka) * v[0] + b[1] * (q[1] @ k[1]) * u2)
        if not (rel_l2(o[0, 0], o1) < 1e-12 and rel_l2(o[1, 0], o2) < 1e-12):
            failed.append(f"two_tokens_{gate}_{l2}")
    # closed form: two tokens, raw gate with softplus arguments around and
    # above the large-argument branch point (30)
    p = tiny_problem(rng, [2], 1, 5, 3, gate="raw")
    p["dt_bias"] = np.zeros((1, 5))
    p["gate"] = np.array([25.0, 29.5, 30.5, 38.0, 45.0])[None, None, :].repeat(2, axis=0)
    p["A_log"] = np.array([-np.log(35.0)])
    o = _run(lib, p)
    q, k, v, b = p["q"][:, 0], p["k"][:, 0], p["v"][:, 0], p["beta"][:, 0]
    a = np.exp(-np.exp(p["A_log"][0]) * np.logaddexp(0.0, p["gate"][:, 0]))
    ka = a[1] * k[0]
    u2 = v[1] - b[0] * (k[1] @ ka) * v[0]
    o2 = 5 ** -0.5 * (b[0] * (q[1] @ ka) * v[0] + b[1] * (q[1] @ k[1]) * u2)
    if not rel_l2(o[1, 0], o2) < 1e-12:
        failed.append("two_tokens_raw_large")
    # finite differences
    for gate, l2 in (("g", False), ("raw", False), ("g", True), ("raw", True)):
        p = tiny_problem(rng, [3, 2], 1, 4, 3, gate=gate, l2norm=l2)
        if not _fd_ok(lib, p):
            failed.append(f"fd_{gate}_{l2}")
    # chunked form
    p = tiny_problem(rng, [11, 6], 1, 5, 4)
    o, S = _run(lib, p, chunk=3)
    oc, Sc = chunked.forward(p["cu"], p["q"], p["k"], p["v"], p["beta"], p["gate"], 5 ** -0.5, 3)
    if not (rel_l2(o, oc) < 1e-12 and rel_l2(S, Sc) < 1e-12):
        failed.append("chunked_fwd")
    gr = _grad(lib, p)
    gc = chunked.backward(p["cu"], p["q"], p["k"], p["v"], p["beta"], p["gate"], p["dO"],
                          5 ** -0.5, 3)
    if not all(rel_l2(gr[n], gc[n]) < 1e-12 for n in gc):
        failed.append("chunked_bwd")
    # a sequence split inside its second document, run fragment by fragment
    # with the state handed over, gives the unsplit outputs and gradients
    from test_oracle_state import split
    p = tiny_problem(rng, [4, 6, 3], 1, 4, 3)
    o, g = _run(lib, p), _grad(lib, p)
    A, B = split(p, 7)
    oA, SA = _run(lib, A, final_state=True)
    oB = _run(lib, B, s_init=SA)
    gB = _grad(lib, B, s_init=SA, ds_final=np.zeros_like(SA))
    gA = _grad(lib, A, ds_final=gB["ds_init"])
    if not rel_l2(np.concatenate([oA, oB]), o) < 1e-12:
        failed.append("split_fwd")
    if not all(rel_l2(np.concatenate([gA[n], gB[n]]), g[n]) < 1e-11
               for n in ("dq", "dk", "dv", "dbeta", "dg")):
        failed.append("split_bwd")
    return failed


@pytest.fixture(scope="module")
def mutant_libs(tmp_path_factory):
    src = open(SRC).read()
    d = tmp_path_factory.mktemp("mutants")
    jobs = {}
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) == 1, f"mutation site of {name} not unique"
        path = os.path.join(d, f"{name}.cpp")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        jobs[name] = path
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        futs = {n: ex.submit(ko.compile_source, p, p[:-4] + ".so") for n, p in jobs.items()}
        return {n: f.result() for n, f in futs.items()}


def test_unmodified_oracle_passes_battery():
    assert battery(None) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, mutant_libs):
    lib = ko.open_library(mutant_libs[name])
    assert battery(lib) != [], f"planted mistake {name} passed every pin"
