"""Pins of the oracle's gradients (CPU only).

The backward oracle is the forward definition differentiated by hand; these
tests tie it to things fixed independently of that derivation:
  * central differences of the forward oracle itself (Richardson-extrapolated,
    on inputs that are multiples of 2^-8 so the +-h perturbations are exact in
    fp32), for every flag combination, both scan conventions and shared angle
    streams;
  * the one-token closed form (softmax weight 1: o = v, so dv = dO and every
    other gradient vanishes);
  * invariance under a common shift of all angles of a pair (scores and the
    transported values only see differences Theta_i - Theta_j), so dL/dTheta
    sums to zero over positions and the inclusive-scan dL/dphi_0 is zero;
  * the column-sum identities of softmax attention: sum_j dL/dv~_j =
    sum_i dL/do~_i and sum_j dL/dk~_j = 0;
  * textbook causal softmax attention (no rotation): the gradients of a
    library autodiff (torch, fp64 CPU).
"""
import numpy as np
import pytest

import oracle

FLAG_SETS = {
    "qk": oracle.ROTATE_QK,
    "qk+v": oracle.ROTATE_QK | oracle.ROTATE_V,
    "qk+v+alibi": oracle.ROTATE_QK | oracle.ROTATE_V | oracle.ALIBI,
    "none": 0,
    "v": oracle.ROTATE_V,
    "qk+v+exclusive": oracle.ROTATE_QK | oracle.ROTATE_V | oracle.SCAN_EXCLUSIVE,
}


def _grid(rng, shape, scale=1.0):
    """fp32 values on the 2^-8 grid (|x| < 4), so x +- 2^-9, 2^-10 are exact."""
    return (np.round(rng.standard_normal(shape) * scale * 256) / 256).clip(-3.9, 3.9).astype(np.float32)


def _problem(seed, B, H, L, d, flags, hphi=None):
    rng = np.random.default_rng(seed)
    q, k, v = (_grid(rng, (B, H, L, d)) for _ in range(3))
    phi = _grid(rng, (B, hphi or H, L, d // 2))
    alibi = np.array([0.5 / (h + 1) for h in range(H)], dtype=np.float32)
    g = rng.standard_normal((B, H, L, d)).astype(np.float32)
    return q, k, v, phi, alibi, g


def _loss(q, k, v, phi, flags, alibi, g):
    o = oracle.Problem(q, k, v, phi, flags, alibi=alibi).output(nthreads=1)
    return float((o * g.astype(np.float64)).sum())


def _numeric(f, x):
    """Richardson-extrapolated central differences of f at every element of x."""
    out = np.zeros(x.shape, dtype=np.float64)
    for idx in np.ndindex(x.shape):
        def cd(h):
            a = x.copy(); a[idx] += np.float32(h)
            b = x.copy(); b[idx] -= np.float32(h)
            return (f(a) - f(b)) / (2 * h)
        d1, d2 = cd(2.0 ** -9), cd(2.0 ** -10)
        out[idx] = (4 * d2 - d1) / 3
    return out


@pytest.mark.parametrize("name", list(FLAG_SETS) + ["shared-phi"])
def test_gradients_match_central_differences(name):
    flags = FLAG_SETS.get(name, oracle.ROTATE_QK | oracle.ROTATE_V)
    hphi = 1 if name == "shared-phi" else None
    q, k, v, phi, alibi, g = _problem(11, 1, 2, 5, 4, flags, hphi)
    got = oracle.Problem(q, k, v, phi, flags, alibi=alibi).backward(g, nthreads=1)
    want = {
        "dq": _numeric(lambda x: _loss(x, k, v, phi, flags, alibi, g), q),
        "dk": _numeric(lambda x: _loss(q, x, v, phi, flags, alibi, g), k),
        "dv": _numeric(lambda x: _loss(q, k, x, phi, flags, alibi, g), v),
        "dphi": _numeric(lambda x: _loss(q, k, v, x, flags, alibi, g), phi),
    }
    for n, w in want.items():
        err = np.abs(got[n] - w).max()
        assert err <= 2e-8 * max(1.0, np.abs(w).max()), f"{name} {n}: max err {err:.3e}"


@pytest.mark.parametrize("name", list(FLAG_SETS))
def test_single_token_closed_form(name):
    flags = FLAG_SETS[name]
    q, k, v, phi, alibi, g = _problem(3, 2, 3, 1, 8, flags)
    got = oracle.Problem(q, k, v, phi, flags, alibi=alibi).backward(g, nthreads=1)
    np.testing.assert_allclose(got["dv"], g.astype(np.float64), rtol=0, atol=1e-13)
    for n in ("dq", "dk", "dphi"):
        assert np.abs(got[n]).max() <= 1e-13, n


@pytest.mark.parametrize("name", list(FLAG_SETS) + ["shared-phi"])
def test_common_angle_shift_invariance(name):
    flags = FLAG_SETS.get(name, oracle.ROTATE_QK | oracle.ROTATE_V)
    hphi = 1 if name == "shared-phi" else None
    q, k, v, phi, alibi, g = _problem(5, 2, 2, 48, 8, flags, hphi)
    got = oracle.Problem(q, k, v, phi, flags, alibi=alibi).backward(g)
    tot = got["dtheta"].sum(axis=2)
    assert np.abs(tot).max() <= 1e-10 * max(1.0, np.abs(got["dtheta"]).max()), tot
    if not flags & oracle.SCAN_EXCLUSIVE:
        assert np.abs(got["dphi"][:, :, 0]).max() <= 1e-10 * max(1.0, np.abs(got["dphi"]).max())


@pytest.mark.parametrize("name", ["qk+v", "qk+v+alibi", "none", "v"])
def test_column_sum_identities(name):
    flags = FLAG_SETS[name]
    q, k, v, phi, alibi, g = _problem(7, 1, 2, 40, 8, flags)
    prob = oracle.Problem(q, k, v, phi, flags, alibi=alibi)
    got = prob.backward(g)
    theta = prob.theta()
    zero = np.zeros_like(theta)
    rv = theta if flags & oracle.ROTATE_V else zero
    rk = theta if flags & oracle.ROTATE_QK else zero
    dv_rot = oracle.rotate_rows(got["dv"].astype(np.float32), rv)
    do_rot = oracle.rotate_rows(g, rv)
    np.testing.assert_allclose(dv_rot.sum(axis=2), do_rot.sum(axis=2), rtol=0, atol=2e-5)
    dk_rot = oracle.rotate_rows(got["dk"].astype(np.float32), rk)
    assert np.abs(dk_rot.sum(axis=2)).max() <= 2e-5


def test_textbook_attention_gradients_match_autodiff():
    torch = pytest.importorskip("torch")
    q, k, v, phi, alibi, g = _problem(9, 2, 2, 33, 8, 0)
    got = oracle.Problem(q, k, v, phi, 0).backward(g)
    Q, K, V = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = Q @ K.transpose(-1, -2) / np.sqrt(8)
    mask = torch.ones(33, 33, dtype=torch.bool).tril()
    s = s.masked_fill(~mask, float("-inf"))
    o = torch.softmax(s, dim=-1) @ V
    (o * torch.tensor(g, dtype=torch.float64)).sum().backward()
    for n, t in (("dq", Q), ("dk", K), ("dv", V)):
        np.testing.assert_allclose(got[n], t.grad.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("flags", [oracle.ROTATE_QK, oracle.ROTATE_QK | oracle.ROTATE_V | oracle.ALIBI],
                         ids=["qk", "qk+v+alibi"])
def test_gate_gradient_matches_central_differences(flags):
    """With the forget gate the backward also returns dL/d(log f_s); it and the
    other gradients against Richardson central differences of the forward
    oracle (log f on the 2^-8 grid, negative, so the perturbed gates stay
    valid log-probabilities)."""
    flags |= oracle.FORGET
    q, k, v, phi, alibi, g = _problem(13, 1, 2, 6, 4, flags)
    rng = np.random.default_rng(14)
    logf = (-np.round(rng.uniform(0.05, 1.5, size=(1, 2, 6)) * 256) / 256).astype(np.float32)

    def loss(q_, k_, v_, phi_, lf_):
        o = oracle.Problem(q_, k_, v_, phi_, flags, alibi=alibi, logf=lf_).output(nthreads=1)
        return float((o * g.astype(np.float64)).sum())

    got = oracle.Problem(q, k, v, phi, flags, alibi=alibi, logf=logf).backward(g, nthreads=1)
    want = {
        "dlogf": _numeric(lambda x: loss(q, k, v, phi, x), logf),
        "dq": _numeric(lambda x: loss(x, k, v, phi, logf), q),
        "dk": _numeric(lambda x: loss(q, x, v, phi, logf), k),
        "dphi": _numeric(lambda x: loss(q, k, v, x, logf), phi),
    }
    for n, w in want.items():
        err = np.abs(got[n] - w).max()
        assert err <= 2e-8 * max(1.0, np.abs(w).max()), f"gate {n}: max err {err:.3e}"
    # log f_0 enters no logit (the route j -> i holds steps j+1..i)
    assert np.all(got["dlogf"][:, :, 0] == 0.0)


def test_gate_gradient_equals_prefix_of_column_sums():
    """Because every causal row of dS sums to zero, dL/d(log f_s) equals the
    sum over t < s of the column sums sum_i dS_it.  Checked on the oracle's
    own dS, rebuilt here from its public row scores (an identity of the
    softmax gradient, independent of how the oracle accumulates dlogf)."""
    flags = oracle.ROTATE_QK | oracle.FORGET
    q, k, v, phi, alibi, g = _problem(15, 1, 1, 7, 4, flags)
    logf = np.full((1, 1, 7), -0.25, dtype=np.float32)
    prob = oracle.Problem(q, k, v, phi, flags, logf=logf)
    got = prob.backward(g, nthreads=1)["dlogf"][0, 0]
    # dS_ij = alpha_ij (<dO~_i, v~_j> - D_i); with no value transport dO~ = dO and
    # v~ = v, and o_i = sum_j alpha_ij v_j
    L = 7
    dS = np.zeros((L, L))
    for i in range(L):
        s = np.array(prob.scores_row(0, 0, i))
        a = np.exp(s - s.max()); a /= a.sum()
        vv = v[0, 0, : i + 1].astype(np.float64)
        gi = g[0, 0, i].astype(np.float64)
        o = a @ vv
        dS[i, : i + 1] = a * (vv @ gi - o @ gi)
    colsum = dS.sum(axis=0)
    want = np.concatenate([[0.0], np.cumsum(colsum)[:-1]])
    assert np.abs(got - want).max() <= 1e-12 * max(1.0, np.abs(want).max())
