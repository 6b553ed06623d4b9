"""Pins of the oracle's forget-gate bias (CPU only).

The bias adds sum_{s=j+1}^{i} log f_s to score (i, j) (the PaTH reading notes'
Sec. 2.5; named beside the distance bias as far-mass control in "Why Do
Accumulated Transformations Extrapolate?" Sec. 4).  Pinned by:
  * constant gates log f_s = -m: the sum is -m (i - j), the distance bias with
    slope m (ALiBi, whose oracle path is pinned on its own);
  * open gates log f = 0: no bias at all;
  * brute force on tiny inputs: attention weights formed as
    exp(scale <q~_i, k~_j>) * prod_{s=j+1}^{i} f_s with the explicit product,
    normalised, then the transported sum.
"""
import numpy as np
import pytest

import oracle

QK, V, AL, FG = oracle.ROTATE_QK, oracle.ROTATE_V, oracle.ALIBI, oracle.FORGET


def _inputs(seed, B=1, H=2, L=40, d=8):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, H, L, d)).astype(np.float32) for _ in range(3))
    phi = (rng.standard_normal((B, H, L, d // 2)) * 0.4).astype(np.float32)
    return q, k, v, phi


@pytest.mark.parametrize("flags", [QK, QK | V, 0])
def test_constant_gates_equal_distance_bias(flags):
    q, k, v, phi = _inputs(1)
    B, H, L, _ = q.shape
    slopes = np.array([0.5, 0.0625], dtype=np.float32)
    logf = np.broadcast_to(-slopes[None, :, None], (B, H, L)).astype(np.float32)
    gated = oracle.attention(q, k, v, phi, flags | FG, logf=logf)
    alibi = oracle.attention(q, k, v, phi, flags | AL, alibi=slopes)
    np.testing.assert_allclose(gated, alibi, rtol=0, atol=1e-12)


def test_open_gates_are_no_bias():
    q, k, v, phi = _inputs(2)
    logf = np.zeros(q.shape[:3], dtype=np.float32)
    np.testing.assert_array_equal(oracle.attention(q, k, v, phi, QK | V | FG, logf=logf),
                                  oracle.attention(q, k, v, phi, QK | V))


@pytest.mark.parametrize("flags", [QK, QK | V, V])
def test_brute_force_gate_products(flags):
    q, k, v, phi = _inputs(3, B=1, H=1, L=7, d=4)
    rng = np.random.default_rng(4)
    f = rng.uniform(0.2, 1.0, size=q.shape[:3])
    logf = np.log(f).astype(np.float32)
    f = np.exp(logf.astype(np.float64))  # the gates the oracle sees
    got = oracle.attention(q, k, v, phi, flags | FG, logf=logf)
    theta = oracle.angle_scan(phi)
    zero = np.zeros_like(theta)
    tq = theta if flags & QK else zero
    tv = theta if flags & V else zero
    qr = oracle.rotate_rows(q, tq)[0, 0]
    kr = oracle.rotate_rows(k, tq)[0, 0]
    vr = oracle.rotate_rows(v, tv)[0, 0]
    L, d = qr.shape
    want = np.zeros((L, d))
    for i in range(L):
        w = np.array([np.exp(qr[i] @ kr[j] / np.sqrt(d)) * np.prod(f[0, 0, j + 1:i + 1])
                      for j in range(i + 1)])
        w /= w.sum()
        o = (w[:, None] * vr[:i + 1]).sum(axis=0)
        want[i] = oracle.rotate_rows(o.astype(np.float32)[None], tv[0, 0, i:i + 1], inverse=True)[0] \
            if flags & V else o
    np.testing.assert_allclose(got[0, 0], want, rtol=0, atol=2e-6)


@pytest.mark.parametrize("kind", ["open", "constant"])
def test_gated_backward_reduces_to_ungated(kind):
    """Open gates leave every gradient of the ungated problem unchanged;
    constant gates -m give the gradients of the distance bias with slope m."""
    q, k, v, phi = _inputs(5, L=12)
    B, H, L, _ = q.shape
    dout = np.random.default_rng(6).standard_normal(q.shape).astype(np.float32)
    slopes = np.array([0.5, 0.0625], dtype=np.float32)
    if kind == "open":
        logf = np.zeros((B, H, L), dtype=np.float32)
        ref = oracle.Problem(q, k, v, phi, QK | V).backward(dout)
    else:
        logf = np.broadcast_to(-slopes[None, :, None], (B, H, L)).astype(np.float32)
        ref = oracle.Problem(q, k, v, phi, QK | V | AL, alibi=slopes).backward(dout)
    got = oracle.Problem(q, k, v, phi, QK | V | FG, logf=logf).backward(dout)
    for n in ("dq", "dk", "dv", "dphi"):
        np.testing.assert_allclose(got[n], ref[n], rtol=0, atol=1e-11, err_msg=n)
    assert got["dlogf"].shape == (B, H, L)
