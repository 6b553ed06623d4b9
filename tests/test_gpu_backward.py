"""GPU parity of the backward pass (bf16) against the fp64 oracle's gradients.

Inputs: the seeded workloads of the forward tests, plus an upstream gradient
dO ~ N(0, 1) rounded to bf16 (seeded).  The oracle differentiates the forward
it defines, in fp64, from the same bf16 bits.

Bars.  dq, dk, dv are bf16 outputs of products whose operands are rounded to
bf16 on the GPU (q~, k~, v~, do~ and the probabilities P and dS); each output
is a sum of many such terms, so the error is relative to the output's own
scale: max |err| <= 2e-2 * max|ref| and rms(err) <= 1e-2 * rms(ref).  dTheta
(fp32) carries the same operand rounding and is held to the same bars.  dphi
is a suffix sum of dTheta over positions: the exact dTheta sums to zero over
positions (the loss is invariant under a common angle shift), so dphi is a
small difference of long sums and carries the accumulated error of every
term summed; it is held to 2e-2 of its own scale for both the maximum and the
rms error.  The forward's lse (fp32) is compared with the oracle's scores on
sampled rows to 1e-3 (base-2 units: a 0.1% error in the softmax scale).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from accumulated_rotation_positional_amd import binding
from accumulated_rotation_positional_amd import workloads as wl
from gpu_util import DEV, oracle_problem, say, to_dev, to_host

pytestmark = pytest.mark.gpu

FLAG_SETS = [
    dict(rotate_qk=True, rotate_v=False, alibi=False),
    dict(rotate_qk=True, rotate_v=True, alibi=False),
    dict(rotate_qk=True, rotate_v=True, alibi=True),
    dict(rotate_qk=False, rotate_v=False, alibi=False),
    dict(rotate_qk=False, rotate_v=True, alibi=False),
    dict(rotate_qk=True, rotate_v=True, alibi=False, exclusive=True),
]
MAX_REL, RMS_REL = 2e-2, 1e-2


def _ids(fs):
    return "-".join(k for k, v in fs.items() if v) or "nope"


def _dout(w, seed=100):
    g = np.random.default_rng(seed).standard_normal((w.batch, w.heads, w.seqlen, w.head_dim))
    return wl.to_bf16_bits(g.astype(np.float32))


def run_backward(w, dout_bits, *, rotate_qk=True, rotate_v=False, alibi=False, exclusive=False):
    say(f"[gpu] backward {w.name} B={w.batch} H={w.heads} L={w.seqlen} d={w.head_dim} "
        f"qk={rotate_qk} v={rotate_v} alibi={alibi} excl={exclusive}")
    q, k, v, phi = to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.phi)
    slopes = w.alibi if w.alibi is not None else wl.alibi_slopes(w.heads)
    al = to_dev(slopes) if alibi else None
    o, theta, lse, desc = binding.forward_train(q, k, v, phi, rotate_qk=rotate_qk,
                                                rotate_v=rotate_v, alibi=al, exclusive=exclusive)
    dq, dk, dv, dphi, dtheta = binding.backward(desc, q, k, v, phi, theta, o, lse,
                                                to_dev(dout_bits), alibi=al)
    torch.cuda.synchronize()
    return dict(dq=to_host(dq), dk=to_host(dk), dv=to_host(dv), dphi=dphi.cpu().numpy(),
                dtheta=dtheta.cpu().numpy(), lse=lse.cpu().numpy())


def assert_grad_close(got, want, what):
    scale = max(float(np.abs(want).max()), 1e-6)
    err = np.abs(got.astype(np.float64) - want)
    rms_ref = float(np.sqrt(np.mean(want ** 2))) or 1e-12
    rms_err = float(np.sqrt(np.mean(err ** 2)))
    say(f"[gpu] {what}: max err {err.max():.3e} (ref max {scale:.3e}), rms err/ref "
        f"{rms_err / rms_ref:.3e}")
    assert np.all(np.isfinite(got)), what
    assert err.max() <= MAX_REL * scale, f"{what}: max err {err.max():.3e} > {MAX_REL} * {scale:.3e}"
    assert rms_err <= RMS_REL * rms_ref, f"{what}: rms err {rms_err:.3e} > {RMS_REL} * {rms_ref:.3e}"


def assert_dphi_close(got, want, what):
    scale = max(float(np.abs(want).max()), 1e-6)
    err = np.abs(got.astype(np.float64) - want)
    rms_ref = float(np.sqrt(np.mean(want ** 2))) or 1e-12
    rms_err = float(np.sqrt(np.mean(err ** 2)))
    say(f"[gpu] {what}: max err {err.max():.3e} (ref max {scale:.3e}), rms err/ref "
        f"{rms_err / rms_ref:.3e}")
    assert np.all(np.isfinite(got)), what
    assert err.max() <= MAX_REL * scale, f"{what}: max err {err.max():.3e} > {MAX_REL} * {scale:.3e}"
    assert rms_err <= MAX_REL * rms_ref, f"{what}: rms err {rms_err:.3e} > {MAX_REL} * {rms_ref:.3e}"


def compare_all(w, flags, got):
    prob = oracle_problem(w, rotate_qk=flags.get("rotate_qk", True),
                          rotate_v=flags.get("rotate_v", False), alibi=flags.get("alibi", False),
                          exclusive=flags.get("exclusive", False))
    want = prob.backward(_dout(w))
    tag = f"{w.name} L={w.seqlen} d={w.head_dim} {_ids(flags)}"
    for n in ("dq", "dk", "dv"):
        assert_grad_close(got[n], want[n], f"{tag} {n}")
    if flags.get("rotate_qk", True) or flags.get("rotate_v", False):
        assert_grad_close(got["dtheta"], want["dtheta"], f"{tag} dtheta")
        assert_dphi_close(got["dphi"], want["dphi"], f"{tag} dphi")
    else:
        assert np.abs(got["dphi"]).max() == 0.0 and np.abs(got["dtheta"]).max() == 0.0


@pytest.mark.parametrize("flags", FLAG_SETS, ids=[_ids(f) for f in FLAG_SETS])
@pytest.mark.parametrize("name,L", [("train_1k", 333), ("rope_8k_d128", 200)])
def test_backward_small_all_flags(name, L, flags):
    w = wl.make(name, batch=2, heads=3, seqlen=L)
    got = run_backward(w, _dout(w), **flags)
    compare_all(w, flags, got)


@pytest.mark.parametrize("L", [2, 31, 64, 65, 257, 700])
@pytest.mark.parametrize("name", ["train_1k", "rope_8k_d128"])
def test_backward_ragged_lengths(name, L):
    w = wl.make(name, batch=1, heads=2, seqlen=L)
    flags = dict(rotate_qk=True, rotate_v=True, alibi=True)
    compare_all(w, flags, run_backward(w, _dout(w), **flags))


@pytest.mark.parametrize("name", ["train_1k", "rope_8k_d128"])
def test_backward_single_token_closed_form(name):
    """L = 1: the softmax weight is 1 and o = v exactly, so dv = dO and every
    other gradient is zero.  On the GPU dS = <do~, v~ - o~> with o~ the bf16
    forward output, so dq, dk and dphi are bounded by the rounding of o:
    |dS| <= |do~| |v~| 2^-8 and |dq|, |dk| <= scale |dS| |k~| (or |q~|)."""
    w = wl.make(name, batch=2, heads=3, seqlen=1)
    dout = _dout(w)
    got = run_backward(w, dout, rotate_qk=True, rotate_v=True, alibi=True)
    g = wl.from_bf16_bits(dout).astype(np.float64)
    assert np.abs(got["dv"] - g).max() <= 2e-2 * np.abs(g).max()
    def nrm(name):
        return float(np.sqrt((w.values(name).astype(np.float64) ** 2).sum(axis=-1)).max())
    d = w.head_dim
    ds_max = float(np.sqrt((g ** 2).sum(axis=-1)).max()) * nrm("v") * 2.0 ** -7
    bound = ds_max * max(nrm("q"), nrm("k")) / np.sqrt(d)
    for n in ("dq", "dk"):
        assert np.abs(got[n]).max() <= bound, (n, np.abs(got[n]).max(), bound)
    assert np.abs(got["dphi"]).max() <= 2 * ds_max + bound * max(nrm("q"), nrm("k")), \
        np.abs(got["dphi"]).max()


def test_backward_shared_angle_heads():
    w = wl.make("train_1k", batch=2, heads=4, seqlen=300)
    w.phi = np.ascontiguousarray(w.phi[:, :1])
    flags = dict(rotate_qk=True, rotate_v=True)
    compare_all(w, flags, run_backward(w, _dout(w), **flags))


def test_backward_two_thousand_tokens():
    w = wl.make("train_1k", batch=1, heads=2, seqlen=2048)
    flags = dict(rotate_qk=True, rotate_v=True)
    compare_all(w, flags, run_backward(w, _dout(w), **flags))


@pytest.mark.parametrize("name", ["train_1k", "rope_8k_d128"])
def test_backward_paired_blocks_match_unpaired(name):
    """64 heads at 2000 tokens: the dQ pass pairs its 256-query blocks (64 x 8
    = 512 blocks, half of them still fill the CUs) and the dK/dV pass its key
    blocks; three of those heads alone pair neither.  A dQ block is computed
    the same way in both, so dq (and the forward's lse) must agree bit for
    bit.  A paired dK/dV workgroup walks its second key block up from the
    diagonal instead of down from the last query tile, so dk, dv, dTheta and
    dphi are the same fp32 sums in another order: each element within one
    bf16 unit in the last place of itself plus 1e-6 of the largest element
    (sums with cancellation)."""
    w = wl.make(name, batch=1, heads=64, seqlen=2000)
    dout = _dout(w)
    flags = dict(rotate_qk=True, rotate_v=True)
    big = run_backward(w, dout, **flags)
    part = dataclasses.replace(w, heads=3, **{n: np.ascontiguousarray(getattr(w, n)[:, :3])
                                              for n in ("q", "k", "v", "phi")})
    small = run_backward(part, np.ascontiguousarray(dout[:, :3]), **flags)
    for key in ("dq", "lse"):
        assert np.array_equal(small[key].view(np.uint32), big[key][:, :3].view(np.uint32)), key
    for key in ("dk", "dv", "dtheta", "dphi"):
        a, b = small[key].astype(np.float64), big[key][:, :3].astype(np.float64)
        m = float(np.abs(b).max())
        excess = np.abs(a - b) - 2.0 ** -7 * np.abs(b)
        say(f"[gpu] paired vs unpaired {key}: max |diff| {np.abs(a - b).max():.3e}, beyond 1 ulp "
            f"{max(float(excess.max()), 0.0) / m:.3e} of max {m:.3e}")
        # measured: at most 3e-8 of the largest element beyond one bf16 unit
        assert float(excess.max()) <= 1e-6 * m, key


@pytest.mark.parametrize("slopes", [(1.0, 0.25), (0.5, -0.002)], ids=["steep", "mixed-sign"])
@pytest.mark.parametrize("name", ["train_1k", "rope_8k_d128"])
def test_backward_steep_distance_bias(name, slopes):
    """With a steep distance bias most (query tile, key range) blocks hold
    only probabilities that are exactly zero in fp32, and both gradient
    kernels start their walks past them.  2048 tokens, every element of dq,
    dk, dv and dtheta against the oracle; one head with a negative slope (far
    keys favoured), for which no block can be left out."""
    w = wl.make(name, batch=1, heads=2, seqlen=2048)
    w.alibi = np.array(slopes, dtype=np.float32)
    flags = dict(rotate_qk=True, rotate_v=True, alibi=True)
    got = run_backward(w, _dout(w), **flags)
    want = oracle_problem(w, rotate_qk=True, rotate_v=True, alibi=True).backward(_dout(w))
    tag = f"{w.name} steep slopes {slopes}"
    for n in ("dq", "dk", "dv", "dtheta"):
        assert_grad_close(got[n], want[n], f"{tag} {n}")
    # dphi_s = sum_{t >= s} dtheta_t.  Under a steep bias the true dphi is a
    # small difference of many dtheta terms, so the bf16-level error of dtheta
    # (checked above) dominates it relative to its own scale; check instead
    # that dphi is the exact suffix sum of the computed dtheta (fp32
    # accumulation over 2048 terms).
    dth = got["dtheta"].astype(np.float64)
    suffix = np.cumsum(dth[:, :, ::-1], axis=2)[:, :, ::-1]
    absum = np.cumsum(np.abs(dth)[:, :, ::-1], axis=2)[:, :, ::-1]
    err = np.abs(got["dphi"] - suffix)
    say(f"[gpu] {tag} dphi vs suffix sums of dtheta: max err {err.max():.3e}")
    assert np.all(err <= 1e-5 * absum + 1e-30)


@pytest.mark.parametrize("name", ["train_1k", "rope_8k_d128"])
def test_forward_train_lse_matches_oracle_scores(name):
    w = wl.make(name, batch=1, heads=2, seqlen=300)
    got = run_backward(w, _dout(w), rotate_qk=True, rotate_v=True)
    prob = oracle_problem(w, rotate_qk=True, rotate_v=True, alibi=False)
    for h in range(2):
        for i in (0, 1, 63, 64, 150, 299):
            s = prob.scores_row(0, h, i)
            m = s.max()
            want = (m + np.log(np.exp(s - m).sum())) / np.log(2.0)
            assert abs(got["lse"][0, h, i] - want) <= 1e-3 * max(1.0, abs(want)), (h, i)


def test_backward_full_size_identities():
    """extrap_16k at full size (B=2, H=8, L=16384, d=64): identities that hold
    at any size -- a common shift of the angles leaves the loss unchanged, so
    dTheta sums to zero over positions (and dphi_0 = 0); the column sums of
    softmax attention: sum_j R(Theta_j) dv_j = sum_i R(Theta_i) dO_i and
    sum_j R(Theta_j) dk_j = 0."""
    w = wl.make("extrap_16k")
    dout = _dout(w)
    flags = dict(rotate_qk=True, rotate_v=True)
    got = run_backward(w, dout, **flags)
    for n in ("dq", "dk", "dv", "dphi", "dtheta"):
        assert np.all(np.isfinite(got[n])), n
    dth = got["dtheta"].astype(np.float64)
    tot = dth.sum(axis=2)
    assert np.all(np.abs(tot) <= 1e-3 * np.abs(dth).sum(axis=2)), np.abs(tot).max()
    # dphi_0 is the same full sum (per angle head and pair), formed by the reverse scan
    assert np.all(np.abs(got["dphi"][:, :, 0]) <= 1e-3 * np.abs(dth).sum(axis=2)), \
        np.abs(got["dphi"][:, :, 0]).max()
    theta = oracle.angle_scan(w.phi)
    dv_rot = oracle.rotate_rows(got["dv"].astype(np.float32), theta)
    do_rot = oracle.rotate_rows(wl.from_bf16_bits(dout), theta)
    lhs, rhs = dv_rot.sum(axis=2), do_rot.sum(axis=2)
    assert np.abs(lhs - rhs).max() <= 2e-2 * np.abs(rhs).max() + 1.0, np.abs(lhs - rhs).max()
    dk_rot = oracle.rotate_rows(got["dk"].astype(np.float32), theta).sum(axis=2)
    assert np.abs(dk_rot).max() <= 2e-2 * np.abs(oracle.rotate_rows(
        got["dk"].astype(np.float32), theta)).sum(axis=2).max(), np.abs(dk_rot).max()
