"""Pins of the FP64 oracle against things other than itself.

The pages print no worked numeric example, so the pins are closed forms the
recurrence must reduce to, central finite differences of L = sum(o*dO),
agreement with an independent chunked formulation (the chunked training form
is an exact re-arrangement of the recurrence), and exact invariants.
Sizes use K != V so a transposed state or a swapped index cannot hide.
"""

import numpy as np
import pytest

from helpers import rel_l2, tiny_problem
from models import kda_chunked_fp64 as chunked
from oracle import kda_oracle as ko


def _fwd(p, **kw):
    return ko.fwd(p["cu"], p["q"], p["k"], p["v"], p["beta"], p["gate"], p.get("A_log"),
                  p.get("dt_bias"), gate_form=p["gate_form"], l2norm=p["l2norm"], **kw)


def _bwd(p, **kw):
    return ko.bwd(p["cu"], p["q"], p["k"], p["v"], p["beta"], p["gate"], p["dO"],
                  p.get("A_log"), p.get("dt_bias"), gate_form=p["gate_form"],
                  l2norm=p["l2norm"], **kw)


def _softplus(x):
    return np.logaddexp(0.0, x)


# ---------------------------------------------------------------- closed forms

def test_single_token():
    """One token from a zero state: o = scale * beta * (q.k) * v."""
    rng = np.random.default_rng(1)
    p = tiny_problem(rng, [1], 1, 6, 5)
    o = _fwd(p)
    s = 6 ** -0.5
    ref = s * p["beta"][0, 0] * (p["q"][0, 0] @ p["k"][0, 0]) * p["v"][0, 0]
    assert rel_l2(o[0, 0], ref) < 1e-13


def test_one_hot_keys_is_linear_attention():
    """k_t = e_t, g = 0, beta = 1: the keys never interfere, so
    o_t = scale * sum_{i<=t} q_t[i] v_i."""
    rng = np.random.default_rng(2)
    K, V, T = 7, 4, 7
    p = tiny_problem(rng, [T], 1, K, V)
    p["k"] = np.eye(K)[:T].reshape(T, 1, K)
    p["gate"] = np.zeros((T, 1, K))
    p["beta"] = np.ones((T, 1))
    o = _fwd(p)
    s = K ** -0.5
    for t in range(T):
        ref = s * sum(p["q"][t, 0, i] * p["v"][i, 0] for i in range(t + 1))
        assert rel_l2(o[t, 0], ref) < 1e-13


def test_repeated_key_overwrites():
    """Same unit key every step, beta = 1, g = 0: the delta rule replaces the
    stored value, so o_t = scale * (q_t.k) * v_t."""
    rng = np.random.default_rng(3)
    K, V, T = 4, 6, 9
    p = tiny_problem(rng, [T], 1, K, V)
    p["k"] = np.full((T, 1, K), 0.5)          # exactly unit norm
    p["gate"] = np.zeros((T, 1, K))
    p["beta"] = np.ones((T, 1))
    o = _fwd(p)
    s = K ** -0.5
    ref = s * (p["q"][:, 0] @ p["k"][0, 0])[:, None] * p["v"][:, 0]
    assert rel_l2(o[:, 0], ref) < 1e-13


def test_total_forgetting():
    """g = -1e4 (exp underflows to 0): each token sees only itself."""
    rng = np.random.default_rng(4)
    p = tiny_problem(rng, [11], 2, 5, 3)
    p["gate"] = np.full_like(p["gate"], -1e4)
    o = _fwd(p)
    s = 5 ** -0.5
    ref = s * (p["beta"] * np.einsum("thc,thc->th", p["q"], p["k"]))[..., None] * p["v"]
    assert rel_l2(o, ref) < 1e-13


def test_beta_zero_gives_zero():
    rng = np.random.default_rng(5)
    p = tiny_problem(rng, [6, 3], 2, 5, 4)
    p["beta"] = np.zeros_like(p["beta"])
    assert np.all(_fwd(p) == 0.0)


def _two_token_ref(q, k, v, beta, a, s):
    """Two tokens from a zero state, written out by hand:
    S1 = b1 k1 v1^T; S2' = Diag(a2) S1; u2 = v2 - S2'^T k2; S2 = S2' + b2 k2 u2^T."""
    ka = a[1] * k[0]
    u2 = v[1] - beta[0] * (k[1] @ ka) * v[0]
    o1 = s * beta[0] * (q[0] @ k[0]) * v[0]
    o2 = s * (beta[0] * (q[1] @ ka) * v[0] + beta[1] * (q[1] @ k[1]) * u2)
    return o1, o2


def test_two_tokens_gate_g():
    """Pins that the decay multiplies the key rows before the delta update."""
    rng = np.random.default_rng(6)
    K, V = 5, 3
    p = tiny_problem(rng, [2], 1, K, V, decay=1.0)
    o = _fwd(p)
    a = np.exp(p["gate"][:, 0])
    o1, o2 = _two_token_ref(p["q"][:, 0], p["k"][:, 0], p["v"][:, 0], p["beta"][:, 0], a, K ** -0.5)
    assert rel_l2(o[0, 0], o1) < 1e-13
    assert rel_l2(o[1, 0], o2) < 1e-13


def test_two_tokens_raw_gate():
    """Raw gate: g = -exp(A_log) * softplus(a + dt_bias), per head and channel."""
    rng = np.random.default_rng(7)
    K, V, H = 5, 3, 2
    p = tiny_problem(rng, [2], H, K, V, gate="raw")
    o = _fwd(p)
    for h in range(H):
        g = -np.exp(p["A_log"][h]) * _softplus(p["gate"][:, h] + p["dt_bias"][h])
        o1, o2 = _two_token_ref(p["q"][:, h], p["k"][:, h], p["v"][:, h], p["beta"][:, h],
                                np.exp(g), K ** -0.5)
        assert rel_l2(o[0, h], o1) < 1e-13
        assert rel_l2(o[1, h], o2) < 1e-13


def _large_argument_problem(seed):
    """Two tokens with the raw gate's softplus argument a + dt_bias in
    [25, 45]: both sides of the oracle's x > 30 branch. A_log = -log(35)
    keeps g = -softplus(x)/35 near -1, so the decay is neither 0 nor 1 and
    softplus(x) ~ x + e^-x is what the output depends on."""
    rng = np.random.default_rng(seed)
    K, V, H = 6, 3, 2
    p = tiny_problem(rng, [2], H, K, V, gate="raw")
    x = rng.uniform(25.0, 45.0, (2, H, K))
    x[:, :, 0], x[:, :, 1] = 29.5, 30.5           # straddle the branch point
    p["dt_bias"] = rng.normal(0.0, 0.5, (H, K))
    p["gate"] = x - p["dt_bias"][None]
    p["A_log"] = np.full(H, -np.log(35.0))
    return p


def test_two_tokens_raw_gate_large_arguments():
    """softplus for a + dt_bias > 30: g = -exp(A_log) * (x + log1p(e^-x)),
    checked against the closed form of two tokens (numpy's logaddexp as
    softplus), and the backward against central differences."""
    p = _large_argument_problem(17)
    o = _fwd(p)
    K = p["q"].shape[2]
    for h in range(p["q"].shape[1]):
        x = p["gate"][:, h] + p["dt_bias"][h]
        assert np.all(x > 24.0) and np.any(x > 30.0) and np.any(x < 30.0)
        g = -np.exp(p["A_log"][h]) * _softplus(x)
        o1, o2 = _two_token_ref(p["q"][:, h], p["k"][:, h], p["v"][:, h], p["beta"][:, h],
                                np.exp(g), K ** -0.5)
        assert rel_l2(o[0, h], o1) < 1e-13
        assert rel_l2(o[1, h], o2) < 1e-13
    g = _bwd(p)
    for inp, out in (("gate", "da"), ("A_log", "dA_log"), ("dt_bias", "ddt_bias")):
        fd = _fd_grad(p, inp, h=1e-5)
        assert rel_l2(g[out], fd) < 1e-6, (inp, rel_l2(g[out], fd))


def test_two_tokens_l2_norm():
    """Fused L2 norm: q <- q (sum q^2 + eps)^-1/2, k likewise, before the rule."""
    rng = np.random.default_rng(8)
    K, V = 6, 4
    p = tiny_problem(rng, [2], 1, K, V, l2norm=True, decay=0.5)
    eps = 1e-6
    o = _fwd(p, l2_eps=eps)
    qn = p["q"][:, 0] / np.sqrt(np.sum(p["q"][:, 0] ** 2, axis=-1, keepdims=True) + eps)
    kn = p["k"][:, 0] / np.sqrt(np.sum(p["k"][:, 0] ** 2, axis=-1, keepdims=True) + eps)
    o1, o2 = _two_token_ref(qn, kn, p["v"][:, 0], p["beta"][:, 0], np.exp(p["gate"][:, 0]),
                            K ** -0.5)
    assert rel_l2(o[0, 0], o1) < 1e-13
    assert rel_l2(o[1, 0], o2) < 1e-13


def test_scale_argument():
    rng = np.random.default_rng(9)
    p = tiny_problem(rng, [5], 1, 4, 4)
    np.testing.assert_allclose(_fwd(p, scale=0.3), _fwd(p, scale=1.0) * 0.3, rtol=1e-14)


# ------------------------------------------------------------ finite differences

def _loss(p, **kw):
    return float(np.sum(_fwd(p, **kw) * p["dO"]))


def _fd_grad(p, name, h=1e-6):
    x = p[name]
    g = np.zeros_like(x)
    flat, gflat = x.reshape(-1), g.reshape(-1)
    for i in range(flat.size):
        old = flat[i]
        flat[i] = old + h
        lp = _loss(p)
        flat[i] = old - h
        lm = _loss(p)
        flat[i] = old
        gflat[i] = (lp - lm) / (2 * h)
    return g


@pytest.mark.parametrize("gate", ["g", "raw"])
@pytest.mark.parametrize("l2norm", [False, True])
def test_backward_matches_finite_differences(gate, l2norm):
    rng = np.random.default_rng(10 + 2 * (gate == "raw") + l2norm)
    p = tiny_problem(rng, [5, 4], 2, 5, 4, gate=gate, l2norm=l2norm)
    g = _bwd(p)
    names = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta",
             "gate": "da" if gate == "raw" else "dg"}
    if gate == "raw":
        names.update(A_log="dA_log", dt_bias="ddt_bias")
    for inp, out in names.items():
        fd = _fd_grad(p, inp)
        err = rel_l2(g[out], fd)
        assert err < 1e-6, (inp, err)


# --------------------------------------------------- chunked form vs recurrence

@pytest.mark.parametrize("C", [1, 3, 64])
def test_chunked_form_agrees(C):
    rng = np.random.default_rng(20 + C)
    p = tiny_problem(rng, [70, 0, 9, 133], 2, 8, 6)
    s = 8 ** -0.5
    o, S = _fwd(p, chunk=C)
    oc, Sc = chunked.forward(p["cu"], p["q"], p["k"], p["v"], p["beta"], p["gate"], s, C)
    assert rel_l2(oc, o) < 1e-12
    assert rel_l2(Sc, S) < 1e-12
    g = _bwd(p)
    gc = chunked.backward(p["cu"], p["q"], p["k"], p["v"], p["beta"], p["gate"], p["dO"], s, C)
    for n in ("dq", "dk", "dv", "dbeta", "dg"):
        assert rel_l2(gc[n], g[n]) < 1e-12, n


def test_chunked_form_agrees_at_head_dim_128():
    rng = np.random.default_rng(30)
    p = tiny_problem(rng, [100, 37], 1, 128, 128)
    s = 128 ** -0.5
    o, S = _fwd(p, chunk=64)
    oc, Sc = chunked.forward(p["cu"], p["q"], p["k"], p["v"], p["beta"], p["gate"], s, 64)
    assert rel_l2(oc, o) < 1e-12 and rel_l2(Sc, S) < 1e-12
    g = _bwd(p)
    gc = chunked.backward(p["cu"], p["q"], p["k"], p["v"], p["beta"], p["gate"], p["dO"], s, 64)
    for n in ("dq", "dk", "dv", "dbeta", "dg"):
        assert rel_l2(gc[n], g[n]) < 1e-12, n


def test_affine_state_map():
    """The state carried across a chunk is an affine function of the incoming
    state (the per-chunk FP32 affine summary S_out = M S_in + B of flashinfer
    PR #7176, opening section). A first token with beta_0 in {0, b, 2b} sets
    S_in = beta_0 k_0 v_0^T; every later state must then move linearly in b."""
    rng = np.random.default_rng(31)
    p = tiny_problem(rng, [11], 1, 6, 5)
    states = []
    for b0 in (0.0, 0.4, 0.8):
        p["beta"][0, 0] = b0
        _, S = _fwd(p, chunk=1)          # state at the start of every token
        states.append(S[1:, 0])
    d1 = states[1] - states[0]
    d2 = states[2] - states[0]
    np.testing.assert_allclose(d2, 2 * d1, rtol=1e-10, atol=1e-13)
    assert np.linalg.norm(d1) > 1e-3


# ----------------------------------------------------------------- invariants

@pytest.mark.parametrize("gate", ["g", "raw"])
def test_euler_identities(gate):
    """o is linear in v, and (without L2 norm) linear in q, so
    sum<v,dv> = sum<q,dq> = sum<o,dO>."""
    rng = np.random.default_rng(40)
    p = tiny_problem(rng, [13, 20], 2, 6, 5, gate=gate)
    L = _loss(p)
    g = _bwd(p)
    assert abs(np.sum(p["v"] * g["dv"]) - L) < 1e-12 * max(1, abs(L))
    assert abs(np.sum(p["q"] * g["dq"]) - L) < 1e-12 * max(1, abs(L))


def test_l2_norm_scale_invariance():
    """With the fused L2 norm, o does not change when q_t or k_t is scaled, so
    <q_t,dq_t> = <k_t,dk_t> = 0 up to the eps term."""
    rng = np.random.default_rng(41)
    p = tiny_problem(rng, [12], 2, 6, 5, l2norm=True)
    g = _bwd(p)
    for x, dx in (("q", "dq"), ("k", "dk")):
        dots = np.einsum("thc,thc->th", p[x], g[dx])
        mags = np.linalg.norm(p[x], axis=-1) * np.linalg.norm(g[dx], axis=-1)
        assert np.all(np.abs(dots) <= 1e-5 * mags + 1e-14)


def test_raw_parameter_gradients_are_sums():
    """ddt_bias[h,c] = sum_t da[t,h,c] (dt_bias enters only through a + dt_bias)."""
    rng = np.random.default_rng(42)
    p = tiny_problem(rng, [7, 9], 3, 5, 4, gate="raw")
    g = _bwd(p)
    np.testing.assert_allclose(g["ddt_bias"], g["da"].sum(axis=0), rtol=1e-12, atol=1e-14)


def test_document_isolation_and_permutation():
    rng = np.random.default_rng(43)
    p = tiny_problem(rng, [9, 14, 5], 2, 5, 4)
    o = _fwd(p)
    g = _bwd(p)
    # perturb document 1: documents 0 and 2 are bitwise unchanged
    p2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
    sl = slice(9, 23)
    for name in ("q", "k", "v", "gate", "dO"):
        p2[name][sl] += 0.1
    p2["beta"][sl] *= 0.5
    o2 = _fwd(p2)
    g2 = _bwd(p2)
    keep = np.r_[0:9, 23:28]
    assert np.array_equal(o[keep], o2[keep])
    for n in g:
        assert np.array_equal(g[n][keep], g2[n][keep]), n
    # permuting the documents permutes the outputs
    order = [2, 0, 1]
    lens = [9, 14, 5]
    starts = [0, 9, 23]
    idx = np.concatenate([np.arange(starts[d], starts[d] + lens[d]) for d in order])
    p3 = {k: (v[idx] if isinstance(v, np.ndarray) and v.ndim >= 2 else v) for k, v in p.items()}
    p3["cu"] = np.concatenate([[0], np.cumsum([lens[d] for d in order])])
    o3 = _fwd(p3)
    assert np.array_equal(o3, o[idx])


def test_heads_are_independent():
    rng = np.random.default_rng(44)
    p = tiny_problem(rng, [10, 6], 3, 5, 4, gate="raw")
    o = _fwd(p)
    g = _bwd(p)
    for h in range(3):
        ph = dict(p)
        for n in ("q", "k", "v", "beta", "gate", "dO"):
            ph[n] = np.ascontiguousarray(p[n][:, h:h + 1])
        ph["A_log"] = p["A_log"][h:h + 1]
        ph["dt_bias"] = p["dt_bias"][h:h + 1]
        np.testing.assert_array_equal(_fwd(ph)[:, 0], o[:, h])
        gh = _bwd(ph)
        for n in ("dq", "dk", "dv", "da"):
            np.testing.assert_array_equal(gh[n][:, 0], g[n][:, h])
        np.testing.assert_allclose(gh["dA_log"][0], g["dA_log"][h], rtol=1e-14)


def test_empty_problem_and_empty_documents():
    rng = np.random.default_rng(45)
    p = tiny_problem(rng, [0, 0], 1, 4, 4)
    assert _fwd(p).shape == (0, 1, 4)
    p = tiny_problem(rng, [0, 5, 0], 1, 4, 4)
    o = _fwd(p)
    q = tiny_problem(rng, [5], 1, 4, 4)
    for n in ("q", "k", "v", "beta", "gate", "dO"):
        q[n] = p[n]
    np.testing.assert_array_equal(_fwd(q), o)


def test_rejects_bad_cu_seqlens():
    rng = np.random.default_rng(46)
    p = tiny_problem(rng, [4, 4], 1, 4, 4)
    p["cu"] = np.array([0, 5, 4])
    with pytest.raises(ValueError):
        _fwd(p)
    p["cu"] = np.array([0, 4, 9])
    with pytest.raises(ValueError):
        _fwd(p)
