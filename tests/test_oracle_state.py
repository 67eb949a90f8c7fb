"""Pins of the oracle's boundary states: a state entering document 0
(s_init), the state leaving the last document (s_final), and in the backward
the gradient with respect to s_final (ds_final) and the one it returns with
respect to s_init (ds_init). These are one rank's share of a sequence split
over ranks (flashinfer PR #7176, opening section: the recurrent state passed
between fragments). Pinned by: a sequence split anywhere and run fragment by
fragment with the state handed over gives the unsplit outputs and gradients;
the decay-only closed form (beta = 0); affinity of s_final in s_init (and
independence from it once a later document starts); central differences for
ds_init and for the inputs' gradients under a nonzero ds_final."""

import numpy as np
import pytest

from helpers import rel_l2, tiny_problem
from oracle import kda_oracle as ko


def _fwd(p, **kw):
    return ko.fwd(p["cu"], p["q"], p["k"], p["v"], p["beta"], p["gate"], p.get("A_log"),
                  p.get("dt_bias"), gate_form=p["gate_form"], l2norm=p["l2norm"], **kw)


def _bwd(p, **kw):
    return ko.bwd(p["cu"], p["q"], p["k"], p["v"], p["beta"], p["gate"], p["dO"],
                  p.get("A_log"), p.get("dt_bias"), gate_form=p["gate_form"],
                  l2norm=p["l2norm"], **kw)


def split(p, m):
    """Fragments [0, m) and [m, T) of a packed problem; a document that
    straddles m continues in the second fragment."""
    cu = p["cu"]
    A, B = dict(p), dict(p)
    for key in ("q", "k", "v", "beta", "gate", "dO"):
        A[key], B[key] = p[key][:m], p[key][m:]
    A["cu"] = np.concatenate([cu[cu < m], [m]]).astype(np.int64)
    B["cu"] = np.concatenate([[0], cu[cu > m] - m]).astype(np.int64)
    return A, B


def grad_names(p):
    return ("dq", "dk", "dv", "dbeta") + (("da",) if p["gate_form"] == "raw" else ("dg",))


@pytest.mark.parametrize("gate,l2norm", [("g", False), ("raw", False), ("g", True)])
@pytest.mark.parametrize("m", [3, 7, 12])
def test_split_sequence_matches_unsplit(gate, l2norm, m):
    """Tokens [0, m) on one rank and [m, T) on the next: the forward hands over
    s_final, the backward ds_init; outputs and gradients are the unsplit ones.
    m = 7 splits between documents, the others inside one."""
    rng = np.random.default_rng(50 + m)
    p = tiny_problem(rng, [4, 3, 6], 2, 5, 4, gate=gate, l2norm=l2norm)
    o = _fwd(p)
    g = _bwd(p)
    A, B = split(p, m)
    # the state is handed over only when a document continues across m
    cont = m not in p["cu"]
    oA, SA = _fwd(A, final_state=True)
    oB = _fwd(B, s_init=SA if cont else None)
    assert rel_l2(np.concatenate([oA, oB]), o) < 1e-13
    gB = _bwd(B, s_init=SA if cont else None, ds_final=np.zeros_like(SA))
    gA = _bwd(A, ds_final=gB["ds_init"] if cont else None)
    for n in grad_names(p):
        assert rel_l2(np.concatenate([gA[n], gB[n]]), g[n]) < 1e-12, n
    if gate == "raw":
        assert rel_l2(gA["dA_log"] + gB["dA_log"], g["dA_log"]) < 1e-12
        assert rel_l2(gA["ddt_bias"] + gB["ddt_bias"], g["ddt_bias"]) < 1e-12


def test_three_fragments():
    rng = np.random.default_rng(60)
    p = tiny_problem(rng, [9], 1, 4, 3)
    o = _fwd(p)
    g = _bwd(p)
    A, BC = split(p, 3)
    B, C = split(BC, 4)
    oA, SA = _fwd(A, final_state=True)
    oB, SB = _fwd(B, s_init=SA, final_state=True)
    oC = _fwd(C, s_init=SB)
    assert rel_l2(np.concatenate([oA, oB, oC]), o) < 1e-13
    gC = _bwd(C, s_init=SB)
    gB = _bwd(B, s_init=SA, ds_final=gC["ds_init"])
    gA = _bwd(A, ds_final=gB["ds_init"])
    for n in grad_names(p):
        assert rel_l2(np.concatenate([gA[n], gB[n], gC[n]]), g[n]) < 1e-12, n


def test_decay_only_closed_form():
    """beta = 0: S_t = Diag(e^(G_t)) s_init with G_t the running sum of g, so
    o_t = scale (Diag(e^(G_t)) s_init)^T q_t and s_final = Diag(e^(G_T)) s_init."""
    rng = np.random.default_rng(61)
    p = tiny_problem(rng, [6], 2, 5, 3)
    p["beta"][:] = 0.0
    s0 = rng.standard_normal((2, 5, 3))
    o, sf = _fwd(p, s_init=s0, final_state=True)
    G = np.cumsum(p["gate"], axis=0)                           # [T, H, K]
    St = np.exp(G)[..., None] * s0[None]                        # [T, H, K, V]
    ref = 5 ** -0.5 * np.einsum("thkv,thk->thv", St, p["q"])
    assert rel_l2(o, ref) < 1e-14
    assert rel_l2(sf, St[-1]) < 1e-14


def test_final_state_is_affine_in_the_initial_state():
    rng = np.random.default_rng(62)
    p = tiny_problem(rng, [7], 1, 4, 3)
    s1, s2 = rng.standard_normal((2, 1, 4, 3))
    f = lambda s: _fwd(p, s_init=s, final_state=True)[1]
    assert rel_l2(f(s1) + f(s2) - f(np.zeros_like(s1)), f(s1 + s2)) < 1e-13
    # a later document starts from zero: its final state does not see s_init
    q = tiny_problem(rng, [4, 5], 1, 4, 3)
    assert np.array_equal(_fwd(q, s_init=s1, final_state=True)[1],
                          _fwd(q, final_state=True)[1])


def _loss(p, s0, dsf):
    o, sf = _fwd(p, s_init=s0, final_state=True)
    return float(np.sum(o * p["dO"]) + np.sum(sf * dsf))


@pytest.mark.parametrize("gate", ["g", "raw"])
def test_state_gradients_by_central_differences(gate):
    rng = np.random.default_rng(63)
    p = tiny_problem(rng, [5], 1, 3, 3, gate=gate)
    s0 = rng.standard_normal((1, 3, 3))
    dsf = rng.standard_normal((1, 3, 3))
    g = _bwd(p, s_init=s0, ds_final=dsf)
    h = 1e-6
    fd = np.zeros_like(s0)
    for i in np.ndindex(s0.shape):
        a, b = s0.copy(), s0.copy()
        a[i] += h
        b[i] -= h
        fd[i] = (_loss(p, a, dsf) - _loss(p, b, dsf)) / (2 * h)
    assert rel_l2(g["ds_init"], fd) < 1e-7
    # the inputs' gradients see ds_final too
    names = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta",
             "gate": "da" if gate == "raw" else "dg"}
    for inp, out in names.items():
        x = p[inp].reshape(-1)
        fdx = np.zeros_like(x)
        for i in range(x.size):
            old = x[i]
            x[i] = old + h
            lp = _loss(p, s0, dsf)
            x[i] = old - h
            lm = _loss(p, s0, dsf)
            x[i] = old
            fdx[i] = (lp - lm) / (2 * h)
        assert rel_l2(g[out].reshape(-1), fdx) < 1e-7, out


def test_empty_last_document_passes_zero():
    """The state leaving an empty last document is that document's entering
    state: zero, or s_init when it is also document 0."""
    rng = np.random.default_rng(64)
    p = tiny_problem(rng, [5, 0], 1, 3, 2)
    s0 = rng.standard_normal((1, 3, 2))
    assert np.all(_fwd(p, s_init=s0, final_state=True)[1] == 0)
    q = tiny_problem(rng, [0], 1, 3, 2)
    assert np.array_equal(_fwd(q, s_init=s0, final_state=True)[1], s0)
    g = _bwd(q, s_init=s0, ds_final=s0)
    assert np.array_equal(g["ds_init"], s0)
