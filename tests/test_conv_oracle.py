"""Pins of the conv1d + SiLU oracle (oracle/conv_oracle.py) against things
other than itself: numpy's convolution routine and the logistic function of
scipy for the forward, central differences for the backward, and the
structure of packed documents and fragments (document isolation; a document
split into two fragments, the second given the first one's last W-1 tokens
as its halo, gives the unsplit result). Planted mistakes in copies of the
oracle must each fail one of these."""

import os
import types

import numpy as np
import pytest
from scipy.special import expit

from helpers import rel_l2
from oracle import conv_oracle as co

W = co.WIDTH
SRC = os.path.join(os.path.dirname(co.__file__), "conv_oracle.py")


def _problem(rng, lens, D, halo=False, bias=True):
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    p = dict(cu=cu, x=rng.standard_normal((T, D)), w=rng.standard_normal((D, W)) * 0.7,
             dy=rng.standard_normal((T, D)),
             b=rng.standard_normal(D) * 0.3 if bias else None,
             halo=rng.standard_normal((W - 1, D)) if halo else None)
    return p


def _np_reference(p):
    """Per document and channel: numpy's full convolution of the document's
    tokens (after the halo for document 0) with the reversed taps, cut to
    the document; then the logistic function."""
    cu, x, w, b, halo = p["cu"], p["x"], p["w"], p["b"], p["halo"]
    T, D = x.shape
    z = np.zeros((T, D))
    for d in range(len(cu) - 1):
        a, e = int(cu[d]), int(cu[d + 1])
        for c in range(D):
            seq = x[a:e, c]
            lead = halo[:, c] if (d == 0 and halo is not None) else np.zeros(W - 1)
            full = np.convolve(np.concatenate([lead, seq]), w[c, ::-1])
            z[a:e, c] = full[W - 1:W - 1 + (e - a)]
    if b is not None:
        z += b[None, :]
    return z * expit(z)


def _fwd(mod, p):
    return mod.conv_silu_fwd(p["cu"], p["x"], p["w"], p["b"], p["halo"])[0]


def _bwd(mod, p):
    return mod.conv_silu_bwd(p["cu"], p["x"], p["w"], p["dy"], p["b"], p["halo"])


@pytest.mark.parametrize("halo", [False, True])
def test_forward_matches_numpy_convolution(halo):
    rng = np.random.default_rng(1 + halo)
    p = _problem(rng, [7, 1, 2, 12], 5, halo=halo)
    assert rel_l2(_fwd(co, p), _np_reference(p)) < 1e-14


def test_current_token_tap_is_silu():
    rng = np.random.default_rng(3)
    p = _problem(rng, [6, 4], 3)
    p["w"] = np.zeros((3, W))
    p["w"][:, W - 1] = 1.0
    z = p["x"] + p["b"][None]
    assert np.allclose(_fwd(co, p), z / (1.0 + np.exp(-z)), rtol=1e-15, atol=0)


def _fd(mod, p, name, h=1e-6):
    x = p[name]
    g = np.zeros_like(x)
    flat, gflat = x.reshape(-1), g.reshape(-1)
    for i in range(flat.size):
        old = flat[i]
        flat[i] = old + h
        lp = float(np.sum(_fwd(mod, p) * p["dy"]))
        flat[i] = old - h
        lm = float(np.sum(_fwd(mod, p) * p["dy"]))
        flat[i] = old
        gflat[i] = (lp - lm) / (2 * h)
    return g


GRADS = {"x": "dx", "w": "dw", "b": "db", "halo": "dhalo"}


def _fd_ok(mod, p, tol=1e-7):
    g = _bwd(mod, p)
    return all(rel_l2(g[out], _fd(mod, p, inp)) < tol for inp, out in GRADS.items()
               if p[inp] is not None)


def test_backward_matches_finite_differences():
    rng = np.random.default_rng(4)
    p = _problem(rng, [5, 2, 6], 3, halo=True)
    g = _bwd(co, p)
    for inp, out in GRADS.items():
        err = rel_l2(g[out], _fd(co, p, inp))
        assert err < 1e-7, (inp, err)


def test_document_isolation():
    rng = np.random.default_rng(5)
    p = _problem(rng, [5, 8, 3], 4, halo=True)
    y0, g0 = _fwd(co, p), _bwd(co, p)
    p["x"][5:13] += rng.standard_normal((8, 4))
    p["dy"][5:13] += rng.standard_normal((8, 4))
    y1, g1 = _fwd(co, p), _bwd(co, p)
    keep = np.r_[0:5, 13:16]
    assert np.array_equal(y0[keep], y1[keep])
    assert np.array_equal(g0["dx"][keep], g1["dx"][keep])
    assert np.array_equal(g0["dhalo"], g1["dhalo"])


@pytest.mark.parametrize("m", [1, 2, 3, 7])
def test_split_document_with_halo_equals_whole(m):
    """A document split after m tokens: fragment B gets as halo the W-1 tokens
    before its start (zero-padded when the document started less than W-1
    tokens earlier); outputs match, dw and db add, and B's dhalo adds into the
    gradient of A's last tokens."""
    rng = np.random.default_rng(6 + m)
    full = _problem(rng, [11], 3)
    x, n = full["x"], 11
    lead = np.concatenate([np.zeros((W - 1, 3)), x[:m]])[-(W - 1):]
    A = dict(full, cu=np.array([0, m]), x=x[:m].copy(), dy=full["dy"][:m].copy(), halo=None)
    B = dict(full, cu=np.array([0, n - m]), x=x[m:].copy(), dy=full["dy"][m:].copy(), halo=lead)
    yA, yB, yF = _fwd(co, A), _fwd(co, B), _fwd(co, full)
    assert rel_l2(np.concatenate([yA, yB]), yF) < 1e-14
    gA, gB, gF = _bwd(co, A), _bwd(co, B), _bwd(co, full)
    assert rel_l2(gA["dw"] + gB["dw"], gF["dw"]) < 1e-13
    assert rel_l2(gA["db"] + gB["db"], gF["db"]) < 1e-13
    dx = np.concatenate([gA["dx"], gB["dx"]])
    k = min(m, W - 1)
    dx[m - k:m] += gB["dhalo"][W - 1 - k:]
    assert rel_l2(dx, gF["dx"]) < 1e-13


# ---------------------------------------------------------------- planted mistakes

MUTANTS = {
    "taps_reversed": ("z += w[:, j][None, :] * _shifted(x, cu, (WIDTH - 1) - j, halo)",
                      "z += w[:, j][None, :] * _shifted(x, cu, j, halo)"),
    "shift_off_by_one": ("out[a + shift:e] = x[a:e - shift]",
                         "out[a + shift:e] = x[a + 1:e - shift + 1] if e - shift + 1 <= e else x[a:e - shift]"),
    "halo_reversed": ("out[t] = halo[(WIDTH - 1) + (t - a) - shift]",
                      "out[t] = halo[shift - 1 - (t - a)]"),
    "halo_all_docs": ("if d == 0 and halo is not None:", "if halo is not None:"),
    "silu_grad_drops_term": ("dz = dy * (s + z * s * (1.0 - s))", "dz = dy * s"),
    "dx_wrong_tap": ("dx[a:e - shift] += w[:, j][None, :] * dz[a + shift:e]",
                     "dx[a:e - shift] += w[:, (WIDTH - 1) - j][None, :] * dz[a + shift:e]"),
    "dhalo_index": ("t = a + i - j", "t = a + j - i"),
    "no_bias": ("z = np.zeros((T, D)) if b is None else", "z = np.zeros((T, D)) if True else"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"conv_oracle_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def battery(mod):
    failed = []
    rng = np.random.default_rng(77)
    for halo in (False, True):
        p = _problem(rng, [6, 2, 5], 3, halo=halo)
        if not rel_l2(_fwd(mod, p), _np_reference(p)) < 1e-13:
            failed.append(f"numpy_{halo}")
        if not _fd_ok(mod, p):
            failed.append(f"fd_{halo}")
    return failed


def test_unmodified_oracle_passes_battery():
    assert battery(co) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    assert battery(_mutant(name)) != [], f"planted mistake {name} passed every pin"
