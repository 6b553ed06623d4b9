"""GPU parity of the backward with forget gates (arp_backward_ex) against the
fp64 oracle's gradients, dL/d(log f) included.

Gates as in the forward's gate tests: log f_t = log sigmoid(z), z ~ N(2, 1)
per (b, h, t) (mostly open), or z ~ N(0, 1) (strong forgetting), seeded.
Bars: dq, dk, dv and dTheta as in the ungated backward, 2e-2 of their own
maximum (rms 1e-2).  dlogf, a sum of many terms of dS that cancel (each row
of dS sums to zero), is held to the ungated dphi bars (2e-2 of its own scale
for the maximum and the rms).  dphi itself: see assert_dphi_bars."""
import numpy as np
import pytest
import torch

import oracle
from accumulated_rotation_positional_amd import binding
from accumulated_rotation_positional_amd import workloads as wl
from gpu_util import oracle_flags, say, to_dev, to_host
from test_gpu_backward import assert_dphi_close, assert_grad_close

pytestmark = pytest.mark.gpu


def _gates(w, seed=21, mean=2.0):
    z = np.random.default_rng(seed).normal(mean, 1.0, size=(w.batch, w.heads, w.seqlen))
    return (-np.logaddexp(0.0, -z)).astype(np.float32)  # log sigmoid(z)


def _dout(w, seed=101):
    g = np.random.default_rng(seed).standard_normal((w.batch, w.heads, w.seqlen, w.head_dim))
    return wl.to_bf16_bits(g.astype(np.float32))


def _slopes(w):
    return w.alibi if w.alibi is not None else wl.alibi_slopes(w.heads)


def run_gated(w, logf, dout_bits, *, rotate_v=False, alibi=False):
    say(f"[gpu] gated backward {w.name} B={w.batch} H={w.heads} L={w.seqlen} d={w.head_dim} "
        f"v={rotate_v} alibi={alibi}")
    q, k, v, phi = to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.phi)
    al = to_dev(_slopes(w)) if alibi else None
    lf = to_dev(logf)
    o, theta, lse = binding.forward_ex(q, k, v, phi, rotate_qk=True, rotate_v=rotate_v, alibi=al,
                                       logf=lf, with_lse=True)
    flags = binding.flags_for(rotate_qk=True, rotate_v=rotate_v, alibi=alibi,
                              shared_phi=phi.shape[1] == 1 and q.shape[1] != 1, forget=True)
    desc = binding.desc_for(q, flags)
    dq, dk, dv, dphi, dtheta, dlogf = binding.backward_ex(desc, q, k, v, phi, theta, o, lse,
                                                          to_dev(dout_bits), alibi=al, logf=lf)
    torch.cuda.synchronize()
    return dict(dq=to_host(dq), dk=to_host(dk), dv=to_host(dv), dphi=dphi.cpu().numpy(),
                dtheta=dtheta.cpu().numpy(), dlogf=dlogf.cpu().numpy())


def oracle_grads(w, logf, dout_bits, rotate_v, alibi):
    prob = oracle.Problem(w.q, w.k, w.v, w.phi, oracle_flags(True, rotate_v, alibi) | oracle.FORGET,
                          alibi=_slopes(w) if alibi else None, logf=logf)
    return prob.backward(dout_bits)


def compare(got, want, tag):
    """Every check runs (and prints its figures) before the first failure is
    raised."""
    fails = []

    def check(fn, *args):
        try:
            fn(*args)
        except AssertionError as e:
            fails.append(str(e))

    for n in ("dq", "dk", "dv", "dtheta"):
        check(assert_grad_close, got[n], want[n], f"{tag} {n}")
    check(assert_dphi_bars, got, want, f"{tag} dphi")
    check(assert_dphi_close, got["dlogf"], want["dlogf"], f"{tag} dlogf")
    if not np.all(got["dlogf"][:, :, 0] == 0.0):  # no logit holds log f_0
        fails.append(f"{tag}: dlogf_0 != 0")
    assert not fails, "\n".join(fails)


def assert_dphi_bars(got, want, what):
    """dphi_s = sum_{t >= s} dTheta_t.  Gates make attention local: only the
    pairs (i, j) with j < s <= i that straddle s add to the exact dphi_s, a
    few near s, while the error of the suffix sum is that of every dTheta_t
    with t >= s, a random walk over up to L terms.  So dphi's error relative
    to its own scale grows with L and the forgetting rate (measured: up to
    2.6% of its maximum at 700 tokens with strong forgetting), and the bar
    is the one that follows from dTheta's: dphi is the suffix sum of the
    computed dTheta up to fp32 accumulation, so its distance from the
    oracle's is at most the suffix sum of |dTheta - dTheta_oracle| (held to
    the bars above) plus that rounding."""
    scale = max(float(np.abs(want["dphi"]).max()), 1e-6)
    err = np.abs(got["dphi"].astype(np.float64) - want["dphi"])
    rms = float(np.sqrt(np.mean(err ** 2)) / (np.sqrt(np.mean(want["dphi"] ** 2)) or 1e-12))
    say(f"[gpu] {what}: max err {err.max():.3e} (ref max {scale:.3e}), rms err/ref {rms:.3e}")
    dth = got["dtheta"].astype(np.float64)
    suffix = np.cumsum(dth[:, :, ::-1], axis=2)[:, :, ::-1]
    absum = np.cumsum(np.abs(dth)[:, :, ::-1], axis=2)[:, :, ::-1]
    assert np.all(np.abs(got["dphi"] - suffix) <= 1e-5 * absum + 1e-30), f"{what}: not the suffix sum"
    derr = np.abs(dth - want["dtheta"])
    walk = np.cumsum(derr[:, :, ::-1], axis=2)[:, :, ::-1]
    assert np.all(err <= walk + 1e-5 * absum + 1e-12), f"{what}: beyond the summed dTheta error"


@pytest.mark.parametrize("alibi", [False, True])
@pytest.mark.parametrize("rotate_v", [False, True])
@pytest.mark.parametrize("name,L", [("train_1k", 333), ("rope_8k_d128", 200)])
def test_gated_backward_small(name, L, rotate_v, alibi):
    w = wl.make(name, batch=2, heads=3, seqlen=L)
    logf, dout = _gates(w), _dout(w)
    got = run_gated(w, logf, dout, rotate_v=rotate_v, alibi=alibi)
    compare(got, oracle_grads(w, logf, dout, rotate_v, alibi), f"gated {name} L={L} v={rotate_v} "
            f"alibi={alibi}")


@pytest.mark.parametrize("L", [1, 65, 257, 700])
@pytest.mark.parametrize("name", ["train_1k", "rope_8k_d128"])
def test_gated_backward_ragged_strong(name, L):
    """Strong forgetting at lengths that leave tiles part-filled.  (At two
    tokens, strong gates leave dS at the rounding level of the bf16 output o,
    the single-token case of the ungated tests, where relative bars on dq and
    dk do not apply.)"""
    w = wl.make(name, batch=1, heads=2, seqlen=L)
    logf, dout = _gates(w, seed=22, mean=0.0), _dout(w)
    got = run_gated(w, logf, dout, rotate_v=True, alibi=True)
    want = oracle_grads(w, logf, dout, True, True)
    if L == 1:  # one logit, holding no gate: every gate gradient is zero
        assert np.all(got["dlogf"] == 0.0)
        return
    compare(got, want, f"gated strong {name} L={L}")


def test_gated_backward_two_thousand_tokens():
    w = wl.make("train_1k", batch=1, heads=2, seqlen=2048)
    logf, dout = _gates(w, seed=23), _dout(w)
    got = run_gated(w, logf, dout, rotate_v=True)
    compare(got, oracle_grads(w, logf, dout, True, False), "gated L=2048")


def test_open_gates_add_exactly_nothing():
    """log f = 0: G = 0, so the gate terms add exact zeros and the gated
    backward reproduces the plain one bit for bit on the same o and lse; its
    dlogf still matches the oracle (the gradient of a gate at 1 is not 0)."""
    w = wl.make("train_1k", batch=1, heads=2, seqlen=300)
    logf = np.zeros((1, 2, 300), dtype=np.float32)
    dout = _dout(w)
    q, k, v, phi = to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.phi)
    lf = to_dev(logf)
    o, theta, lse = binding.forward_ex(q, k, v, phi, rotate_v=True, logf=lf, with_lse=True)
    gated = binding.backward_ex(binding.desc_for(q, binding.flags_for(rotate_v=True, forget=True)),
                                q, k, v, phi, theta, o, lse, to_dev(dout), logf=lf)
    plain = binding.backward_ex(binding.desc_for(q, binding.flags_for(rotate_v=True)),
                                q, k, v, phi, theta, o, lse, to_dev(dout))
    torch.cuda.synchronize()
    assert plain[5] is None
    for a, b, n in zip(gated[:5], plain[:5], ("dq", "dk", "dv", "dphi", "dtheta")):
        assert torch.equal(a, b), n
    want = oracle_grads(w, logf, dout, True, False)
    assert_dphi_close(gated[5].cpu().numpy(), want["dlogf"], "open gates dlogf")


def test_gates_above_one_are_taken_as_one():
    """The forward takes log f > 0 as 0; the gradient there is 0 and every
    other gradient is that of the clamped gates."""
    w = wl.make("train_1k", batch=1, heads=2, seqlen=200)
    logf = _gates(w, seed=24, mean=0.0)
    raised = logf.copy()
    raised[:, :, 7::5] = np.float32(0.25)
    dout = _dout(w)
    got = run_gated(w, raised, dout, rotate_v=True)
    assert np.all(got["dlogf"][:, :, 7::5] == 0.0)
    clamped = np.minimum(raised, np.float32(0.0))
    want = oracle_grads(w, clamped, dout, True, False)
    keep = np.ones(200, dtype=bool)
    keep[7::5] = False
    want["dlogf"] = want["dlogf"] * keep
    compare(got, want, "gates above one")


def test_plain_backward_rejects_gates():
    w = wl.make("train_1k", batch=1, heads=1, seqlen=64)
    q = to_dev(w.q)
    desc = binding.desc_for(q, binding.flags_for(forget=True))
    lse = torch.zeros(1, 1, 64, dtype=torch.float32, device=q.device)
    with pytest.raises(binding.ArpError) as e:
        binding.backward(desc, q, q, q, to_dev(w.phi), to_dev(w.phi), q, lse, q)
    assert e.value.status == binding.ERR_INVALID_ARG
