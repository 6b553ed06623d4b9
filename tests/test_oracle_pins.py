"""Pins for the fp64 CPU oracle: checks against what the pages and the
mathematics fix, each by a route other than the oracle's own formula.

Sources:
  [ACC]  "Why Do Accumulated Transformations Extrapolate?"
  [ADA]  "AdaRoPE: Not All Attention Heads Should Rotate and Scale Equally"
  [POST] "The RoPE decay curve everyone plots is noise ..." (dev.to)

What each pin would catch is noted on it: a dropped term, a wrong sign on the
sine, the wrong route endpoints (inclusive vs exclusive), a missing value
un-rotation, a mask that drops or adds the diagonal, a bias of the wrong sign.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from accumulated_rotation_positional_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
QK, V, AL, EXCL = oracle.ROTATE_QK, oracle.ROTATE_V, oracle.ALIBI, oracle.SCAN_EXCLUSIVE


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _small_problem(seed, B=1, H=2, L=10, d=8, shared_phi=False, phi_scale=math.pi):
    rng = _rng(seed)
    q = rng.standard_normal((B, H, L, d)).astype(np.float32)
    k = rng.standard_normal((B, H, L, d)).astype(np.float32)
    v = rng.standard_normal((B, H, L, d)).astype(np.float32)
    hphi = 1 if shared_phi else H
    phi = rng.uniform(-phi_scale, phi_scale, size=(B, hphi, L, d // 2)).astype(np.float32)
    alibi = wl.alibi_slopes(H)
    return q, k, v, phi, alibi


# ---------------------------------------------------------------------------
# Rotation: sign and orthogonality
# ---------------------------------------------------------------------------

def test_rotation_matches_complex_multiplication():
    """[POST] "How it is checked": the pair (a, b) rotated by angle t is the
    complex product (a + ib) e^{it}; [ADA] eq. (1) writes the same map as
    G = [[cos, -sin], [sin, cos]].  A sign slip on the sine term fails here."""
    rng = _rng(11)
    x = rng.standard_normal((7, 16)).astype(np.float32)
    ang = rng.uniform(-20, 20, size=(7, 8))
    z = x[:, 0::2].astype(np.float64) + 1j * x[:, 1::2].astype(np.float64)
    for inverse, sign in ((False, 1.0), (True, -1.0)):
        w = z * np.exp(1j * sign * ang)
        want = np.empty((7, 16))
        want[:, 0::2], want[:, 1::2] = w.real, w.imag
        got = oracle.rotate_rows(x, ang, inverse=inverse)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def test_rotation_is_orthogonal_with_unit_determinant():
    """[POST]: R^T R = I and det R = +1; norms of every pair are preserved."""
    rng = _rng(12)
    d = 12
    ang = rng.uniform(-50, 50, size=d // 2)
    eye = np.eye(d, dtype=np.float32)
    # Column c of R is R applied to basis vector e_c.
    R = oracle.rotate_rows(eye, np.tile(ang, (d, 1))).T
    np.testing.assert_allclose(R.T @ R, np.eye(d), atol=1e-14)
    for p in range(d // 2):
        blk = R[2 * p:2 * p + 2, 2 * p:2 * p + 2]
        assert abs(np.linalg.det(blk) - 1.0) < 1e-14
    x = rng.standard_normal((5, d)).astype(np.float32)
    y = oracle.rotate_rows(x, rng.uniform(-9, 9, size=(5, d // 2)))
    xn = np.hypot(x[:, 0::2].astype(np.float64), x[:, 1::2].astype(np.float64))
    yn = np.hypot(y[:, 0::2], y[:, 1::2])
    np.testing.assert_allclose(yn, xn, rtol=1e-14)


def test_rope_shift_invariance_of_scores():
    """[POST] "The identity, in one line" (42 offset/shift combinations up to a
    shift of 4000, worst deviation 1e-15) and [ADA] eq. (2): after RoPE the
    score depends on positions only through their difference."""
    rng = _rng(13)
    d = 16
    theta = np.power(10000.0, -2.0 * np.arange(d // 2) / d)
    q = rng.standard_normal(d).astype(np.float32)
    k = rng.standard_normal(d).astype(np.float32)
    worst = 0.0
    for m, n in [(0, 0), (5, 2), (100, 37), (511, 0), (1000, 999), (7, 3)]:
        base = oracle.rotate_rows(q, m * theta) @ oracle.rotate_rows(k, n * theta)
        for shift in (1, 2, 10, 100, 1000, 2500, 4000):
            s = oracle.rotate_rows(q, (m + shift) * theta) @ oracle.rotate_rows(k, (n + shift) * theta)
            worst = max(worst, abs(s - base))
    assert worst < 1e-12


# ---------------------------------------------------------------------------
# Angle scan
# ---------------------------------------------------------------------------

def test_scan_impulse_gives_exact_step():
    """One nonzero step angle at (t0, p0): the accumulated angle is a step at t0
    (inclusive route [ACC] eq. (6)), or at t0 + 1 for the exclusive variant."""
    L, P, t0, p0 = 40, 6, 13, 4
    phi = np.zeros((3, L, P), dtype=np.float32)
    phi[1, t0, p0] = 0.5
    th = oracle.angle_scan(phi)
    want = np.zeros((3, L, P))
    want[1, t0:, p0] = 0.5
    assert np.array_equal(th, want)
    the = oracle.angle_scan(phi, exclusive=True)
    want_e = np.zeros((3, L, P))
    want_e[1, t0 + 1:, p0] = 0.5
    assert np.array_equal(the, want_e)


def test_scan_of_constant_angle_is_rope():
    """[ADA] Sec. 2.1: a constant step theta_p gives the position-indexed angle.
    Inclusive accumulation over 0-based rows: Theta_t = (t + 1) theta_p, with
    theta_p the fp32 value actually fed in (an fp64 theta would differ by up
    to 5e-4 rad at t = 8192)."""
    d, L = 128, 8192
    theta32 = np.power(10000.0, -2.0 * np.arange(d // 2) / d).astype(np.float32)
    phi = np.broadcast_to(theta32, (1, L, d // 2)).copy()
    th = oracle.angle_scan(phi)[0]
    want = np.arange(1, L + 1, dtype=np.float64)[:, None] * theta32.astype(np.float64)[None, :]
    np.testing.assert_allclose(th, want, rtol=1e-13, atol=1e-13)


def test_rope_post_worked_angles():
    """[POST] NTK section table: slowest pair of a 16-dim head at positions 512
    and 4096 is 0.162 and 1.295 rad; theta_0 = 1.  Read from the oracle's scan
    of constant step angles (Theta after `pos` steps)."""
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "rope_post_angles.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 3
    for d, base, pair, pos, angle, dec in rows:
        d, pair, pos, dec = int(d), int(pair), int(pos), int(dec)
        theta = np.float32(float(base) ** (-2.0 * pair / d))
        phi = np.full((1, pos, 1), theta, dtype=np.float32)
        got = oracle.angle_scan(phi)[0, pos - 1, 0]
        assert round(float(got), dec) == pytest.approx(float(angle), abs=0.5 * 10 ** -dec)
        assert f"{got:.{dec}f}" == angle


def test_wrap_range_and_congruence():
    xs = np.array([0.0, math.pi, -math.pi, 3 * math.pi / 2, -3 * math.pi / 2, 1e4, -1e4,
                   2 * math.pi, 7.0, -7.0, math.nextafter(math.pi, 0), 8191.5])
    w = oracle.wrap(xs)
    assert np.all(w >= -math.pi) and np.all(w < math.pi)
    k = (xs - w) / (2 * math.pi)
    np.testing.assert_allclose(k, np.round(k), atol=1e-9)
    assert w[1] == -math.pi and w[2] == -math.pi
    assert w[3] == pytest.approx(-math.pi / 2, abs=1e-15)
    assert w[4] == pytest.approx(math.pi / 2, abs=1e-15)


def test_wrap_is_exact_and_in_range_at_any_magnitude():
    """wrap(x) = x - k * two_pi exactly (two_pi the double nearest 2 pi, k an
    integer), checked in exact rational arithmetic, and inside [-pi, pi) up to
    the largest doubles."""
    from fractions import Fraction
    rng = np.random.default_rng(11)
    xs = np.concatenate([rng.uniform(-1e6, 1e6, 200), rng.standard_normal(50) * 10.0 ** 12,
                         [1e30, -1e30, 1.7e308, -1.7e308, 2.0 ** 60 + 3.0, -(2.0 ** 53) - 2.0,
                          math.nextafter(math.pi, 0), -math.pi, 5e-324]])
    w = oracle.wrap(xs)
    assert np.all(w >= -math.pi) and np.all(w < math.pi)
    two_pi = Fraction(2.0 * math.pi)
    for x, r in zip(xs, w):
        k = (Fraction(float(x)) - Fraction(float(r))) / two_pi
        assert k.denominator == 1, (x, r)


# ---------------------------------------------------------------------------
# Attention: brute-force route products, textbook reductions, closed forms
# ---------------------------------------------------------------------------

def _block_rot(angles):
    """Dense block-diagonal matrix with 2x2 blocks [[cos, -sin], [sin, cos]]."""
    d = 2 * len(angles)
    M = np.zeros((d, d))
    for p, a in enumerate(angles):
        c, s = math.cos(a), math.sin(a)
        M[2 * p:2 * p + 2, 2 * p:2 * p + 2] = [[c, -s], [s, c]]
    return M


def _brute_force(q, k, v, phi, flags, scale, alibi):
    """[ACC] eq. (6): P_{j->i} = M_{j+1} ... M_i (identity when j = i) as an
    explicit product of dense per-token step matrices, each step a rotation by
    minus its angle ([ACC] App. B.2, H_t = e^{-i psi_t}; App. B.8, position-only
    P_{i-k->i} = R(-omega k)).  The exclusive variant moves the route to steps
    j .. i-1.  Scores [ACC] eq. (8) + bias, softmax eq. (11), aggregation eq. (4)."""
    B, H, L, d = q.shape
    out = np.zeros((B, H, L, d))
    for b in range(B):
        for h in range(H):
            ph = phi[b, 0 if phi.shape[1] == 1 else h].astype(np.float64)
            steps = [_block_rot(ph[t]).T for t in range(L)]
            for i in range(L):
                routes = []
                for j in range(i + 1):
                    Pm = np.eye(d)
                    lo, hi = (j, i - 1) if flags & EXCL else (j + 1, i)
                    for t in range(lo, hi + 1):
                        Pm = Pm @ steps[t]
                    routes.append(Pm if flags & QK or flags & V else None)
                s = np.empty(i + 1)
                for j in range(i + 1):
                    Pq = routes[j] if flags & QK else np.eye(d)
                    s[j] = scale * q[b, h, i].astype(np.float64) @ Pq @ k[b, h, j].astype(np.float64)
                    if flags & AL:
                        s[j] -= float(alibi[h]) * (i - j)
                a = np.exp(s - s.max())
                a /= a.sum()
                acc = np.zeros(d)
                for j in range(i + 1):
                    vj = v[b, h, j].astype(np.float64)
                    acc += a[j] * (routes[j] @ vj if flags & V else vj)
                out[b, h, i] = acc
    return out


@pytest.mark.parametrize("flags", [QK, QK | V, QK | V | AL, QK | AL, V, QK | EXCL, QK | V | EXCL, 0])
@pytest.mark.parametrize("shared_phi", [False, True])
def test_oracle_matches_brute_force_route_products(flags, shared_phi):
    q, k, v, phi, alibi = _small_problem(21 + flags, L=9, d=6, shared_phi=shared_phi)
    scale = 1.0 / math.sqrt(6)
    got = oracle.attention(q, k, v, phi, flags, scale=scale, alibi=alibi)
    want = _brute_force(q, k, v, phi, flags, scale, alibi)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_oracle_matches_brute_force_bf16_inputs():
    """bf16 inputs are read as the exact values of their bit patterns."""
    q, k, v, phi, alibi = _small_problem(31, B=2, H=1, L=8, d=4)
    qb, kb, vb = (wl.to_bf16_bits(x) for x in (q, k, v))
    got = oracle.attention(qb, kb, vb, phi, QK | V | AL, alibi=alibi[:1])
    want = _brute_force(wl.from_bf16_bits(qb), wl.from_bf16_bits(kb), wl.from_bf16_bits(vb),
                        phi, QK | V | AL, 0.5, alibi[:1])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_nope_is_textbook_causal_attention():
    """[ADA] NoPE reduction (theta = 0) and the causal multi-head attention of
    its eq. (4)-(5): compare with torch's scaled_dot_product_attention in fp64."""
    q, k, v, phi, _ = _small_problem(41, B=2, H=3, L=33, d=16)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).double(), torch.from_numpy(k).double(), torch.from_numpy(v).double(),
        is_causal=True).numpy()
    np.testing.assert_allclose(oracle.attention(q, k, v, phi, 0), ref, atol=1e-12, rtol=0)
    zero = np.zeros_like(phi)
    np.testing.assert_allclose(oracle.attention(q, k, v, zero, QK | V), ref, atol=1e-12, rtol=0)


def _rope_relative_reference(q, k, v, theta, scale, rotate_v):
    """[ADA] eq. (8): s_ij = scale * sum_f (q_{2f}, q_{2f+1}) G_{j-i}(theta_f) (k_{2f}, k_{2f+1})^T,
    with G_m(t) = [[cos mt, -sin mt], [sin mt, cos mt]]; values, when
    transported, follow [ACC] App. B.8: P_{i-k->i} = R(-omega k)."""
    L, d = q.shape
    out = np.zeros((L, d))
    for i in range(L):
        s = np.zeros(i + 1)
        for j in range(i + 1):
            m = j - i
            for f in range(d // 2):
                c, sn = math.cos(m * theta[f]), math.sin(m * theta[f])
                G = np.array([[c, -sn], [sn, c]])
                s[j] += q[i, 2 * f:2 * f + 2] @ G @ k[j, 2 * f:2 * f + 2]
        s *= scale
        a = np.exp(s - s.max())
        a /= a.sum()
        for j in range(i + 1):
            vj = v[j].astype(np.float64)
            if rotate_v:
                vj = _block_rot(-(i - j) * theta) @ vj
            out[i] += a[j] * vj
    return out


@pytest.mark.parametrize("rotate_v", [False, True])
def test_constant_angles_reduce_to_closed_form_rope(rotate_v):
    rng = _rng(51)
    L, d = 24, 8
    theta32 = np.power(10000.0, -2.0 * np.arange(d // 2) / d).astype(np.float32) * np.float32(7.0)
    q = rng.standard_normal((1, 1, L, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, L, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, L, d)).astype(np.float32)
    phi = np.broadcast_to(theta32, (1, 1, L, d // 2)).copy()
    flags = QK | (V if rotate_v else 0)
    got = oracle.attention(q, k, v, phi, flags)[0, 0]
    want = _rope_relative_reference(q[0, 0], k[0, 0], v[0, 0], theta32.astype(np.float64),
                                    1.0 / math.sqrt(d), rotate_v)
    np.testing.assert_allclose(got, want, atol=1e-12, rtol=0)


@pytest.mark.parametrize("flags", [QK, QK | V, QK | V | AL])
def test_output_invariant_to_a_global_angle_offset(flags):
    """Adding a constant c_p to every accumulated angle (here: to the first step)
    leaves every route, hence every output, unchanged ([ACC] eq. (6): routes
    hold only steps j+1..i; [POST] shift identity)."""
    q, k, v, phi, alibi = _small_problem(61, B=1, H=2, L=40, d=8)
    base = oracle.attention(q, k, v, phi, flags, alibi=alibi)
    phi2 = phi.copy()
    phi2[:, :, 0, :] += np.float32(2.75)
    # phi2[...,0,:] is an fp32 sum; the offset actually applied is its exact difference.
    np.testing.assert_allclose(oracle.attention(q, k, v, phi2, flags, alibi=alibi), base,
                               atol=1e-12, rtol=0)


def test_zero_query_gives_uniform_weights():
    """q = 0: every score is 0, so the causal softmax is uniform over the i + 1
    keys j <= i and o_i is the running mean of v (no value transport)."""
    _, k, v, phi, _ = _small_problem(71, B=1, H=2, L=30, d=8)
    q = np.zeros_like(k)
    got = oracle.attention(q, k, v, phi, QK)
    want = np.cumsum(v.astype(np.float64), axis=2) / np.arange(1, 31)[None, None, :, None]
    np.testing.assert_allclose(got, want, atol=1e-14, rtol=0)


def test_zero_query_with_value_transport_constant_angles():
    """q = 0 and constant angles: o_i = (1/(i+1)) sum_{n=0..i} R(-n omega) v_{i-n}
    ([ACC] App. B.8), evaluated with complex numbers per pair."""
    rng = _rng(72)
    L, d = 25, 6
    omega = np.array([0.3, 1.1, -2.0], dtype=np.float32)
    v = rng.standard_normal((1, 1, L, d)).astype(np.float32)
    q = np.zeros_like(v)
    phi = np.broadcast_to(omega, (1, 1, L, d // 2)).copy()
    got = oracle.attention(q, rng.standard_normal(v.shape).astype(np.float32), v, phi, QK | V)[0, 0]
    z = v[0, 0, :, 0::2].astype(np.float64) + 1j * v[0, 0, :, 1::2].astype(np.float64)
    om = omega.astype(np.float64)
    for i in range(L):
        n = np.arange(i + 1)[:, None]
        w = (z[i - n[:, 0]] * np.exp(-1j * n * om)).sum(axis=0) / (i + 1)
        np.testing.assert_allclose(got[i, 0::2], w.real, atol=1e-14)
        np.testing.assert_allclose(got[i, 1::2], w.imag, atol=1e-14)


def test_zero_query_with_distance_bias_is_geometric():
    """q = 0 with the bias -m_h (i - j): weights r^{i-j} / sum_{n<=i} r^n with
    r = e^{-m_h}, the normaliser being the geometric series (1 - r^{i+1})/(1 - r)."""
    _, k, v, phi, alibi = _small_problem(73, B=1, H=3, L=20, d=4)
    q = np.zeros_like(k)
    got = oracle.attention(q, k, v, phi, QK | AL, alibi=alibi)
    for h in range(3):
        r = math.exp(-float(alibi[h]))
        for i in range(20):
            w = r ** (i - np.arange(i + 1)) * (1 - r) / (1 - r ** (i + 1))
            np.testing.assert_allclose(got[0, h, i], w @ v[0, h, :i + 1].astype(np.float64),
                                       atol=1e-14)


def test_matched_score_is_mean_route_cosine():
    """[ACC] App. B.6: with every q and k block equal to the same unit 2-vector
    scaled by 1/sqrt(B), the score is (1/B) sum_b cos of the route angle, the
    route angle being the sum of the steps j+1..i of block b."""
    rng = _rng(81)
    L, d = 30, 8
    Bk = d // 2
    # unit vectors whose 1/sqrt(B) = 1/2 multiples are exact in fp32
    for u in (np.array([1.0, 0.0]), np.array([0.0, -1.0])):
        _matched_score_case(rng, L, d, Bk, u)


def _matched_score_case(rng, L, d, Bk, u):
    qv = np.tile(u / math.sqrt(Bk), Bk).astype(np.float32)
    q = np.broadcast_to(qv, (1, 1, L, d)).copy()
    phi = rng.uniform(-1.5, 1.5, size=(1, 1, L, Bk)).astype(np.float32)
    prob = oracle.Problem(q, q.copy(), q.copy(), phi, QK, scale=1.0)
    for i in (0, 1, 7, 29):
        s = prob.scores_row(0, 0, i)
        for j in range(i + 1):
            route = phi[0, 0, j + 1:i + 1].astype(np.float64).sum(axis=0)
            assert s[j] == pytest.approx(np.cos(route).mean(), abs=1e-13)


@pytest.mark.parametrize("flags", [QK, QK | V, QK | V | AL])
def test_first_row_is_first_value(flags):
    """Row 0 attends only to itself: o_0 = v_0 (transport over the empty route is I)."""
    q, k, v, phi, alibi = _small_problem(91, B=2, H=2, L=5, d=8)
    got = oracle.attention(q, k, v, phi, flags, alibi=alibi)
    np.testing.assert_allclose(got[:, :, 0], v[:, :, 0], atol=1e-15, rtol=0)


def test_rows_api_matches_full_output_and_causality():
    """Row selection returns the same rows as the full output; outputs of rows
    <= i do not change when keys, values or angles after i change."""
    q, k, v, phi, alibi = _small_problem(95, B=2, H=2, L=32, d=8)
    prob = oracle.Problem(q, k, v, phi, QK | V | AL, alibi=alibi)
    full = prob.output()
    rows = np.array([0, 5, 31, 32 + 7, 3 * 32 + 31])
    np.testing.assert_array_equal(prob.rows(rows), full.reshape(-1, 8)[rows])
    k2, v2, phi2 = k.copy(), v.copy(), phi.copy()
    k2[:, :, 20:] += 1.0
    v2[:, :, 20:] -= 2.0
    phi2[:, :, 20:] += 0.3
    other = oracle.attention(q, k2, v2, phi2, QK | V | AL, alibi=alibi)
    np.testing.assert_array_equal(other[:, :, :20], full[:, :, :20])
    assert not np.allclose(other[:, :, 20:], full[:, :, 20:])


def test_huge_logits_saturate_to_the_best_key():
    """Softmax in the limit of a large logit scale: all weight on the
    highest-scoring key (no overflow, no NaN).  Catches a softmax that does not
    subtract the row maximum before exponentiating."""
    q, k, v, phi, _ = _small_problem(97, B=1, H=2, L=24, d=8)
    scale = 2000.0
    got = oracle.attention(q, k, v, phi, 0, scale=scale)
    assert np.all(np.isfinite(got))
    for h in range(2):
        for i in range(24):
            s = q[0, h, i].astype(np.float64) @ k[0, h, :i + 1].astype(np.float64).T
            top = np.sort(s)[::-1]
            if i > 0 and (top[0] - top[1]) * scale < 40:
                continue  # near-tie: weights not one-hot
            np.testing.assert_allclose(got[0, h, i], v[0, h, int(np.argmax(s))], atol=1e-15)
