"""Pins of the packed-varlen causal GQA attention oracle (oracle/attn_oracle.py)
against things other than itself: torch's scaled_dot_product_attention and
logsumexp in float64 with an explicit bottom-right causal mask per segment,
closed forms (one key; a zero query averages the visible values), central
differences for the backward, GQA as multi-head attention over repeated key
heads, and segment isolation. Planted mistakes in copies of the oracle must
each fail one of these."""

import os
import types

import numpy as np
import pytest
import torch

from helpers import rel_l2
from oracle import attn_oracle as ao

SRC = os.path.join(os.path.dirname(ao.__file__), "attn_oracle.py")


def _problem(rng, lq, lk, Hq=4, Hkv=2, D=8):
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    return dict(cu_q=cu_q, cu_k=cu_k, q=rng.standard_normal((Tq, Hq, D)),
                k=rng.standard_normal((Tk, Hkv, D)), v=rng.standard_normal((Tk, Hkv, D)),
                dO=rng.standard_normal((Tq, Hq, D)))


def _fwd(mod, p, **kw):
    return mod.attn_fwd(p["cu_q"], p["cu_k"], p["q"], p["k"], p["v"], **kw)


def _bwd(mod, p):
    return mod.attn_bwd(p["cu_q"], p["cu_k"], p["q"], p["k"], p["v"], p["dO"])


def _torch_reference(p):
    """Per segment and head: torch SDPA (float64, CPU) with the bottom-right
    causal mask written as a boolean matrix; lse by torch.logsumexp."""
    q, k, v = (torch.from_numpy(p[x]) for x in ("q", "k", "v"))
    Tq, Hq, D = q.shape
    grp = Hq // k.shape[1]
    o = torch.zeros_like(q)
    lse = torch.full((Tq, Hq), float("-inf"), dtype=torch.float64)
    for s in range(len(p["cu_q"]) - 1):
        a, b = int(p["cu_q"][s]), int(p["cu_q"][s + 1])
        c, e = int(p["cu_k"][s]), int(p["cu_k"][s + 1])
        if b == a or e == c:
            continue
        off = (e - c) - (b - a)
        mask = torch.arange(e - c)[None, :] <= torch.arange(b - a)[:, None] + off
        rows = mask.any(dim=1)
        for h in range(Hq):
            qs, ks, vs = q[a:b, h][rows], k[c:e, h // grp], v[c:e, h // grp]
            if len(qs) == 0:
                continue
            o[a:b, h][rows] = torch.nn.functional.scaled_dot_product_attention(
                qs[None], ks[None], vs[None], attn_mask=mask[rows][None])[0]
            sc = (qs @ ks.T) * D ** -0.5
            lse[a:b, h][rows] = torch.logsumexp(sc.masked_fill(~mask[rows], float("-inf")), dim=1)
    return o.numpy(), lse.numpy()


@pytest.mark.parametrize("lq,lk", [([5, 7, 1], [9, 7, 4]), ([6, 3], [2, 3])])
def test_forward_matches_torch_sdpa(lq, lk):
    """Includes a segment with more queries than keys: its first rows see no
    key (o = 0, lse = -inf)."""
    p = _problem(np.random.default_rng(1), lq, lk)
    o, lse = _fwd(ao, p)
    oref, lref = _torch_reference(p)
    assert rel_l2(o, oref) < 1e-13
    fin = np.isfinite(lref)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.allclose(lse[fin], lref[fin], rtol=1e-13, atol=0)
    assert np.all(o[~fin] == 0)


def test_one_key_closed_form():
    p = _problem(np.random.default_rng(2), [1], [1], Hq=2, Hkv=1)
    o, lse = _fwd(ao, p)
    for h in range(2):
        assert np.allclose(o[0, h], p["v"][0, 0], rtol=1e-15)
        assert np.isclose(lse[0, h], (p["q"][0, h] @ p["k"][0, 0]) * 8 ** -0.5, rtol=1e-14)


def test_zero_query_averages_visible_values():
    p = _problem(np.random.default_rng(3), [4], [6], Hq=1, Hkv=1)
    p["q"][:] = 0.0
    o, lse = _fwd(ao, p)
    for i in range(4):
        n = i + 2 + 1                    # keys 0 .. i + (6 - 4)
        assert np.allclose(o[i, 0], p["v"][:n, 0].mean(axis=0), rtol=1e-14)
        assert np.isclose(lse[i, 0], np.log(n), rtol=1e-15)


def _fd(mod, p, name, h=1e-6):
    x = p[name]
    g = np.zeros_like(x)
    flat, gflat = x.reshape(-1), g.reshape(-1)
    for i in range(flat.size):
        old = flat[i]
        flat[i] = old + h
        lp = float(np.sum(_fwd(mod, p)[0] * p["dO"]))
        flat[i] = old - h
        lm = float(np.sum(_fwd(mod, p)[0] * p["dO"]))
        flat[i] = old
        gflat[i] = (lp - lm) / (2 * h)
    return g


def _fd_ok(mod, p, tol=1e-7):
    g = _bwd(mod, p)
    return all(rel_l2(g["d" + n], _fd(mod, p, n)) < tol for n in ("q", "k", "v"))


def test_backward_matches_finite_differences():
    p = _problem(np.random.default_rng(4), [4, 3], [5, 2], Hq=4, Hkv=2, D=4)
    g = _bwd(ao, p)
    for n in ("q", "k", "v"):
        err = rel_l2(g["d" + n], _fd(ao, p, n))
        assert err < 1e-7, (n, err)


def test_gqa_is_mha_over_repeated_key_heads():
    p = _problem(np.random.default_rng(5), [6, 4], [8, 4], Hq=6, Hkv=2)
    o, _ = _fwd(ao, p)
    g = _bwd(ao, p)
    rep = dict(p, k=np.repeat(p["k"], 3, axis=1), v=np.repeat(p["v"], 3, axis=1))
    o2, _ = _fwd(ao, rep)
    g2 = _bwd(ao, rep)
    assert rel_l2(o, o2) < 1e-14
    assert rel_l2(g["dq"], g2["dq"]) < 1e-13
    for n in ("dk", "dv"):
        assert rel_l2(g[n], g2[n].reshape(g2[n].shape[0], 2, 3, -1).sum(axis=2)) < 1e-13


def test_segment_isolation():
    rng = np.random.default_rng(6)
    p = _problem(rng, [5, 6, 3], [5, 9, 4])
    o0, g0 = _fwd(ao, p)[0], _bwd(ao, p)
    p["q"][5:11] += rng.standard_normal(p["q"][5:11].shape)
    p["k"][5:14] += rng.standard_normal(p["k"][5:14].shape)
    o1, g1 = _fwd(ao, p)[0], _bwd(ao, p)
    keep_q, keep_k = np.r_[0:5, 11:14], np.r_[0:5, 14:18]
    assert np.array_equal(o0[keep_q], o1[keep_q])
    assert np.array_equal(g0["dq"][keep_q], g1["dq"][keep_q])
    assert np.array_equal(g0["dk"][keep_k], g1["dk"][keep_k])


# ---------------------------------------------------------------- planted mistakes

MUTANTS = {
    "mask_strict": ("return j <= i + (Lk - Lq)", "return j < i + (Lk - Lq)"),
    "mask_top_left": ("return j <= i + (Lk - Lq)", "return j <= i"),
    "group_map": ("        for h in range(Hq):\n            g = h // grp\n            S = scale",
                  "        for h in range(Hq):\n            g = h % Hkv\n            S = scale"),
    "no_scale": ("scale = D ** -0.5 if scale is None else scale\n    o = np.zeros",
                 "scale = 1.0 if scale is None else scale\n    o = np.zeros"),
    "delta_wrong": ("delta = np.sum(dO[a:b, h] * o[a:b, h], axis=1, keepdims=True)",
                    "delta = np.sum(dO[a:b, h] * dO[a:b, h], axis=1, keepdims=True)"),
    "dq_no_scale": ("dq[a:b, h] = scale * dS @ k[c:e, g]", "dq[a:b, h] = dS @ k[c:e, g]"),
    "dk_uses_P": ("dk[c:e, g] += scale * dS.T @ q[a:b, h]", "dk[c:e, g] += scale * P.T @ q[a:b, h]"),
    "dv_overwrite": ("dv[c:e, g] += P.T @ dO[a:b, h]", "dv[c:e, g] = P.T @ dO[a:b, h]"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"attn_oracle_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def battery(mod):
    failed = []
    rng = np.random.default_rng(99)
    p = _problem(rng, [5, 4, 2], [7, 4, 1], Hq=4, Hkv=2, D=4)
    o, lse = _fwd(mod, p)
    oref, lref = _torch_reference(p)
    fin = np.isfinite(lref)
    if not (rel_l2(o, oref) < 1e-12 and np.allclose(lse[fin], lref[fin], rtol=1e-12)):
        failed.append("torch")
    if not _fd_ok(mod, p):
        failed.append("fd")
    return failed


def test_unmodified_oracle_passes_battery():
    assert battery(ao) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    assert battery(_mutant(name)) != [], f"planted mistake {name} passed every pin"
